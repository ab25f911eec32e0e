// HIP kernels of the self-speculative decoding round (gfx950, wave64, MFMA).
//
// One self-speculative round (GravityOCR review, section 3.2; velog review,
// round description) is two forward passes of the same decoder plus an
// accept step:
//   draft  : rows [x0, [M] x B] at positions p..p+B; the boundary row sees
//            keys <= p, the mask rows see keys <= p+B (cache + whole window);
//   verify : rows [a0, d1..dB] at positions p+1..p+B+1, causal, overwriting
//            the KV slots the draft wrote for the masks;
//   accept : A = longest prefix with d_j == a_j, commit a0, d1..dA, a(A+1).
// Every visibility rule on the path is "row r sees key j iff j <= lim[r]",
// so one attention kernel serves prefill, AR steps, draft and verify.
//
// Batch-1 decode forwards are latency bound: every kernel here issues all of
// its global loads up front (one dependent memory round trip), and no kernel
// synchronizes with another workgroup; kernel boundaries are the only
// cross-workgroup synchronization.
#include "ssb_device.h"

#include <hip/hip_ext.h>

namespace ssb {

// Timing hook: while set, the next launch carries this start/stop event pair on its dispatch.
hipEvent_t g_prof_ev[2] = {nullptr, nullptr};

#define SSB_LAUNCH(K, G, B, SHM, ST, ...)                                                            \
  do {                                                                                               \
    if (g_prof_ev[0]) hipExtLaunchKernelGGL(K, G, B, SHM, ST, g_prof_ev[0], g_prof_ev[1], 0, __VA_ARGS__); \
    else hipLaunchKernelGGL(K, G, B, SHM, ST, __VA_ARGS__);                                          \
  } while (0)

// ---------------------------------------------------------------------------
// Weight packing: W[N][K] -> tiles [n_tile][k_step][lane][16 bytes].  Lane l
// of (tile t, step s) holds packed row 16t + l%16 and K values
// s*kStepK + (kStepK/4)*(l/16) ... +kStepK/4, so one wave reads 1 KiB of
// contiguous memory per step and feeds it straight to the matrix core.
// Packed-row -> source-row maps (tile row r = packed row % 16, j = tile):
//   mode 0: identity; rows >= n0 are zero padding;
//   mode 1 (q|k|v): head hh = j / (hd/16), jj = j % (hd/16); r < 8 holds head
//           dim 8jj + r, r >= 8 holds dim hd/2 + 8jj + (r-8), so each rotary
//           pair (i, i + hd/2) sits in rows (r, r+8) of one tile;
//   mode 2 (gate|up): r < 8 holds gate row 8j + r, r >= 8 holds up row 8j + r-8.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_pack(uint4* dst, int n_tiles, int K, int mode, const T* src0, const T* src1,
                       const T* src2, int n0, int n1, int hd, int* range_err) {
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  const int ksteps = K / KS;
  const size_t total = (size_t)n_tiles * ksteps * kWave;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < total;
       f += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(f % kWave);
    const size_t ts = f / kWave;
    const int step = (int)(ts % ksteps);
    const int tile = (int)(ts / ksteps);
    const int r = lane % 16;
    const int k = step * KS + PER * (lane / 16);
    const T* src = nullptr;
    int srow = 0;
    if (mode == 0) {
      srow = tile * 16 + r;
      if (srow < n0) src = src0;
    } else if (mode == 1) {
      const int tph = hd / 16;
      const int hh = tile / tph, jj = tile % tph;
      const int dim = r < 8 ? 8 * jj + r : hd / 2 + 8 * jj + (r - 8);
      const int nq = n0 / hd, nk = n1 / hd;
      if (hh < nq) { src = src0; srow = hh * hd + dim; }
      else if (hh < nq + nk) { src = src1; srow = (hh - nq) * hd + dim; }
      else { src = src2; srow = (hh - nq - nk) * hd + dim; }
    } else {
      src = r < 8 ? src0 : src1;
      srow = 8 * tile + (r % 8);
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src) v = *reinterpret_cast<const uint4*>(src + (size_t)srow * K + k);
    if constexpr (sizeof(T) == 2) {
      // bf16 weights are stored as fp16, the matrix cores' operand type for fp16 activations (RNE;
      // exact for magnitudes in [2^-17, 65504]); a value beyond fp16's range is reported
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
      bool big = false;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        big |= fabsf(__uint_as_float(wv[i] << 16)) > 65504.f || fabsf(__uint_as_float(wv[i] & 0xffff0000u)) > 65504.f;
      if (big) *range_err = 1;
      v = bf8_to_h8(v);
    }
    dst[f] = v;
  }
}

// ---------------------------------------------------------------------------
// Row preparation + embedding gather.  Writes the per-row metadata of a
// forward (token, position, visibility limit, request), the fp32 residual
// h = E[token] (or a prefix-embedding row), the first GEMM's input
// xg = h * attn_norm gain (in T) and per-16-column sums of squares of h.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void window_row(const PrepArgs& a, int m, int& tok, int& pos, int& lim,
                                           int& req) {
  if (a.mode == PREP_PREFILL) {
    tok = -1; pos = a.pos0 + m; lim = pos; req = 0;
  } else if (a.mode == PREP_TOKENS) {
    tok = a.tokens[m]; pos = a.pos0 + m; lim = pos; req = 0;
  } else {
    const ReqArgs& ra = *a.req;
    const int W = ra.B + 1;
    const int r = m / W, j = m % W;
    req = r;
    const int p = ra.p[r];
    if (a.mode == PREP_DRAFT) {
      // draft window: boundary x0 at p (causal), masks at p+1..p+B (see the window)
      tok = j == 0 ? ra.x0[r] : (ra.win[r] ? ra.win[r][j - 1] : a.mask_id);
      pos = p + j;
      lim = j == 0 ? p : p + ra.B;
      if (tok < 0 || tok >= a.vocab) tok = a.mask_id;   // keep the gather in bounds
    } else {
      // verify window [a0, d1..dB] at p+1..p+B+1, causal; row j of the draft
      // predicted a0 (j = 0) or d_j
      pos = p + 1 + j;
      lim = pos;
      tok = ra.win[r] ? ra.win[r][j] : a.am_prev[m];
      if (j >= 1 && !ra.win[r]) {
        int pl = -1;
        if (ra.planted[r]) {
          pl = ra.planted[r][j - 1];
        } else if (ra.cont[r]) {
          const int idx = ra.cont_c[r] + j;             // 0-based index of y_{c+1+j}
          const int as = ra.astar[r];
          if (idx < ra.cont_len[r]) {
            if (j <= as) pl = ra.cont[r][idx];
            else if (j == as + 1) pl = (ra.cont[r][idx] + 1) % (a.vocab - 1);
          }
        }
        if (pl >= 0 && pl < a.vocab) tok = pl;
      }
      // an argmax of NaN logits is -1: keep the gather in bounds (the host rejects the round)
      if (tok < 0 || tok >= a.vocab) tok = a.mask_id;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(64) void k_prep_embed(PrepArgs a) {
  const int m = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  stamp_begin(a.stamp);
  int tok, pos, lim, req;
  window_row(a, m, tok, pos, lim, req);
  if (g == 0 && t == 0) {
    a.row_tok[m] = tok; a.row_pos[m] = pos; a.row_lim[m] = lim; a.row_req[m] = req;
    a.row_slot[m] = a.req->pt[req][pos / kPage] * kPage + pos % kPage;
  }
  if (g == 0 && t < a.half) a.row_cs[(size_t)m * a.half + t] = a.rope[(size_t)pos * a.half + t];
  // page ids of each request of the forward, gathered once for every layer's attention
  const int n_req = (a.mode == PREP_DRAFT || a.mode == PREP_VERIFY) ? a.req->n : 1;
  if (g == 1 && m < n_req) {
    const int32_t* pt = a.req->pt[m];
    const int npg = a.req->npg[m];
    for (int i = t; i < a.pt_ld; i += 64) a.fwd_pt[(size_t)m * a.pt_ld + i] = i < npg ? pt[i] : 0;
  }
  const int col = g * 64 + t;
  const T* src = tok >= 0 ? reinterpret_cast<const T*>(a.embed) + (size_t)tok * a.hidden
                          : reinterpret_cast<const T*>(a.prefix) + (size_t)pos * a.hidden;
  const float v = Ty<T>::to_f(src[col]);
  a.h[(size_t)m * a.hidden + col] = v;
  reinterpret_cast<T*>(a.xg)[a.xpk ? pk_off(m, col, a.hidden) : (size_t)m * a.hidden + col] =
      Act<T>::from_f(v * a.gain[col]);
  float s = v * v;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
  if (t % 16 == 0) a.ssq[(size_t)m * a.ssq_ld + col / 16] = s;
  stamp_end(a.stamp);
}

struct Top2 { float v1; int i1; float v2; };

// (written with selects only, so that it compiles to conditional moves rather than branches)
__device__ __forceinline__ Top2 merge_top2(Top2 a, Top2 b) {
  const bool nan = a.i1 == -1 || b.i1 == -1;
  const bool bw = b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1);
  const float v1 = bw ? b.v1 : a.v1;
  const int i1 = bw ? b.i1 : a.i1;
  const float v2 = bw ? fmaxf(a.v1, b.v2) : fmaxf(a.v2, b.v1);
  return Top2{nan ? NAN : v1, nan ? -1 : i1, nan ? NAN : v2};
}
// The record of another lane of the same 8-lane group, moved by DPP (CTRL: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1] or row_half_mirror); merging with it three times, in that order, leaves the
// merge of all 8 lanes in every lane (merge_top2 is associative and commutative).
template <int CTRL>
__device__ __forceinline__ Top2 dpp_top2(Top2 x) {
  return Top2{__int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x.v1), CTRL, 0xF, 0xF, false)),
              __builtin_amdgcn_update_dpp(0, x.i1, CTRL, 0xF, 0xF, false),
              __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x.v2), CTRL, 0xF, 0xF, false))};
}

// ---------------------------------------------------------------------------
// GEMM with fused epilogues:  out[m][n] = sum_k X[m][k] W[n][k].
// Grid (n_tiles / NT, S, m_blocks).  A workgroup owns NT 16-column tiles for
// 16*MT rows and one of S equal K ranges; it has NT*KSL waves.  With many rows
// (a batched round) the looped form runs one workgroup per tile group over a
// stride of row blocks, keeping its weight fragments in registers; each row
// block goes through exactly the per-element operations of the one-block form.  Wave
// w = t*KSL + j reduces K steps [j*KPW, (j+1)*KPW) of the range for tile t
// with an MFMA chain in K order.  The workgroup issues every global load it
// needs before its first MFMA: the weight fragments of each wave, the
// activation slab (rows x K range, staged once in LDS and shared by all
// waves), the norm partials and the inputs of its epilogue.  The KSL partial
// tiles of a tile are added one after another in slice order through LDS.
// The decomposition depends only on K and the GEMM, never on M or MT, so a
// row's value never depends on how many rows share the launch.
// Workgroups stream disjoint weight slices spread over every CU (one CU
// alone pulls only ~20-25 GB/s from HBM on this chip).
// RMSNorm inputs arrive as X = h * gain (in T) and each output row is scaled
// by 1/rms(h), rms from the per-16-column sums of squares added in column
// order (review section 3.1: both modes share these layers).
// ---------------------------------------------------------------------------
// SiLU g / (1 + e^-g): e^-g as 2^(-g log2 e) from the hardware base-2 exponential and the quotient
// as g times the hardware reciprocal (each within about 1 ulp); every kernel uses this one form.
__device__ __forceinline__ float silu_f(float g) {
#pragma clang fp contract(off)
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}

// Sum over aligned groups of g lanes (g a power of two, 1..64), result in every lane of the
// group.  Steps: swap within pairs, within quads (DPP quad permutes), mirror within 8 and 16
// lanes (DPP row half-mirror and mirror), then pairs 16 and 32 apart by lane swaps (xor16_sum,
// xor32_sum).  The pattern is fixed, so the rounding of the sum is too.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int moved;
  const int iv = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: moved = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false); break;    // quad_perm [1,0,3,2]
    case 1: moved = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false); break;    // quad_perm [2,3,0,1]
    case 2: moved = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xF, 0xF, false); break;   // row_half_mirror
    default: moved = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xF, 0xF, false); break;  // row_mirror
  }
  return v + __int_as_float(moved);
}
// Lane l's value paired with lane l ^ 16 (resp. l ^ 32) by a VALU lane swap instead of an LDS
// permute: v_permlane16_swap / v_permlane32_swap of v with itself leave each lane the pair
// {v[l & ~16], v[l | 16]} (resp. 32), lower lane first.  A sum or max of the pair equals
// v + v[l ^ 16] (max, and addition, are commutative).
__device__ __forceinline__ float xor16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// The value of lane l ^ 32 (the same swap, the half that is not the lane's own).
__device__ __forceinline__ float xor32_get(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((int)(threadIdx.x % kWave) < 32 ? p[1] : p[0]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float lane_group_sum(float v, int g) {
  if (g >= 2) v = dpp_add(v, 0);
  if (g >= 4) v = dpp_add(v, 1);
  if (g >= 8) v = dpp_add(v, 2);
  if (g >= 16) v = dpp_add(v, 3);
  if (g >= 32) v = xor16_sum(v);
  if (g >= 64) v = xor32_sum(v);
  return v;
}

// Residual epilogue of a [MB x 16*NT] output tile held in LDS (row stride 17): h += tile,
// next input xg = h * gain_next, per-16-column sums of squares of h.  s_pre holds the
// prefetched h tile [NT][MB][16] and the next gain [NT*16].
// Device-coherent (agent-scope) stores and loads: written through to, and read from, the memory
// side, so another workgroup of the same kernel on another XCD sees them after a grid barrier
// with no cache flush (the workgroup that stores waits for their completion before arriving).
template <typename V>
__device__ __forceinline__ void st_coh(V* p, V v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename V>
__device__ __forceinline__ V ld_coh(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int kCoh = 16;   // cache-policy bit sc1 of a buffer load: device-coherent

template <typename T, int MB, bool COH = false>
__device__ __forceinline__ void resid_epilogue(const GemmArgs& a, float* ctile, const float* s_pre, int tg, int NT,
                                               int m_base, int m_end) {
#pragma clang fp contract(off)
  const float* s_h = s_pre;
  const float* s_g = s_pre + NT * MB * 16;
  for (int e = threadIdx.x; e < NT * MB * 16; e += kGemmThreads) {
    const int t = e / (MB * 16), r = (e / 16) % MB, n = e % 16;
    const int m = m_base + r;
    float* ct = ctile + (t * MB + r) * 17;
    const float v = s_h[e] + ct[n];
    ct[n] = v;
    if (m >= m_end) continue;
    const int col = (tg * NT + t) * 16 + n;
    T* xo = reinterpret_cast<T*>(a.xg_out) + (size_t)m * a.hidden + col;
    if constexpr (COH) {
      st_coh(a.h + (size_t)m * a.hidden + col, v);
      st_coh(xo, Act<T>::from_f(v * s_g[t * 16 + n]));
    } else {
      a.h[(size_t)m * a.hidden + col] = v;
      *xo = Act<T>::from_f(v * s_g[t * 16 + n]);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NT * MB; e += kGemmThreads) {
    const int t = e / MB, r = e % MB;
    const int m = m_base + r;
    if (m >= m_end) continue;
    const float* ct = ctile + (t * MB + r) * 17;
    float sum = 0.f;
    for (int n = 0; n < 16; ++n) sum += ct[n] * ct[n];
    if constexpr (COH) st_coh(a.ssq_out + (size_t)m * a.ssq_ld + tg * NT + t, sum);
    else a.ssq_out[(size_t)m * a.ssq_ld + tg * NT + t] = sum;
  }
}

template <typename T, int MT, int EPI, int KPW, bool MLOOP>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs a) {
  // No multiply-add contraction anywhere in this kernel: both of its forms (one row block per
  // workgroup, or several) then compute exactly the written operations for every row.
#pragma clang fp contract(off)
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int MB = MT * 16;
  constexpr int NTH = kGemmThreads;
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LOGITS);
  constexpr int SB = 12;                            // slab fragments per thread in the first batch
  const int NT = a.NT, KSL = a.KSL;
  const int KR = KSL * KPW * KS;                    // K range of one workgroup
  const int XSTR = KR * (int)sizeof(T) + 16;        // LDS row stride of the slab
  const GemmLds L = gemm_lds(MT, KR * (int)sizeof(T), NT, KSL, a.n_ssq, EPI);
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* slab = smem;
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + L.red);
  float* ctile = reinterpret_cast<float*>(smem + L.ctile);
  __shared__ float s_inv[MB];

  // Single-block form: one row block (blockIdx.z); the LM head's workgroups are persistent over
  // tile groups.  Looped form (MLOOP): one tile group per workgroup, which keeps its weight
  // fragments in registers and walks the row blocks blockIdx.z, blockIdx.z + gridDim.z, ...,
  // loading the next block's slab while the current one is multiplied.
  constexpr bool LOOP = (EPI == EPI_LOGITS) && !MLOOP;
  // DIRECT (one row block, one tile per workgroup, short K slices: QKV and O): no two waves share
  // a K slice of the activations, so each wave loads its own MFMA operand fragments straight into
  // registers (same bounded buffer resource) and the slab is not staged in LDS.  (O: 6.5 -> 6.0 us;
  // the down projection's 16-step slices, 16 rows of 64 B per load, measured 0.4 us slower.)
  constexpr bool DIRECT =
      !MLOOP && !LOOP && KPW <= 4 && (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_PARTIAL);
  int tg = blockIdx.x;
  const int split = blockIdx.y;
  int mb = blockIdx.z;
  // DIRECT GEMMs balance their row blocks (ceil(M / blocks) rows each, at most MB): at 33 rows in
  // 16-row tiles 11 + 11 + 11 rows instead of 16 + 16 + 1, so no wave loads a full block's rows
  // (QKV 7.2 -> 7.0 us).  A block's rows past its end read as zero and are left to the block that
  // owns them.  (The down projection, which stages the whole slab anyway, measured slower so.)
  const int rpb = DIRECT ? min(MB, (a.M + (int)gridDim.z - 1) / (int)gridDim.z) : MB;
  int m_base = mb * rpb;
  int m_end = min(a.M, m_base + rpb);
  const int m_blocks = (a.M + MB - 1) / MB;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool cwave = wave < NT * KSL;               // waves past NT*KSL only help with loads
  const int ksl = wave % KSL;
  const int tsub = cwave ? wave / KSL : 0;
  const int ksteps = a.K / KS;
  const int kstep0 = split * (KSL * KPW) + ksl * KPW;
  const int m_last = a.M - 1;

  stamp_begin(a.stamp);
  // ---- every global load of the prologue is issued before the first wait ----
  // 1. this wave's weight fragments (HBM)
  uint4 wf[KPW];
  {
    const uint4* wp = a.W + ((size_t)(tg * NT + tsub) * ksteps + kstep0) * kWave + lane;
#pragma unroll
    for (int s = 0; s < KPW; ++s) wf[s] = wp[(size_t)s * kWave];
  }
  // 2. activation slab (rows x K range) through a buffer resource bounded at row M: rows past M
  //    read as zero without a memory request
  const int FPR = KR / PER;                         // 16-byte fragments per slab row (a power of two)
  const int fsh = 31 - __builtin_clz(FPR);          // e / FPR == e >> fsh (no integer division)
  const int total = MB * FPR;
  const T* xb = reinterpret_cast<const T*>(a.x) + split * KR;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.x), (short)0,
                                        (DIRECT ? m_end : a.M) * a.ldx * (int)sizeof(T), kBufWord3);
  // a 16-row slab of a 4096-long K range (the down projection) has 8192 fragments: 16 per thread
  constexpr int SBX = SB + ((MT == 1 && KPW == 16) ? 4 : 0);
  uint4 xs[SBX];
  auto load_slab = [&](int mbase) {
#pragma unroll
    for (int b = 0; b < SBX; ++b) {
      const int e = min((int)threadIdx.x + b * NTH, total - 1);
      const int off = ((mbase + (e >> fsh)) * a.ldx + split * KR + (e & (FPR - 1)) * PER) * (int)sizeof(T);
      xs[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
  };
  uint4 bx[DIRECT ? KPW : 1][DIRECT ? MT : 1];
  if constexpr (DIRECT) {
#pragma unroll
    for (int s = 0; s < KPW; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int off = ((m_base + mt * 16 + lane % 16) * a.ldx + (kstep0 + s) * KS + PER * (lane / 16)) *
                        (int)sizeof(T);
        bx[s][mt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
  } else {
    load_slab(m_base);
  }
  // 3. norm partials: G = n_ssq/4 lanes per row, one float4 each, up to 3 passes of rows
  constexpr int NPASS = 3;
  float4 sv[NPASS];
  const int G = a.n_ssq / 4, gsh = 31 - __builtin_clz(G), RP = NTH >> gsh;   // G is a power of two
  const __amdgpu_buffer_rsrc_t sr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.ssq), (short)0, a.M * a.ssq_ld * 4, kBufWord3);
  auto load_norm = [&](int mbase, float4 (&dst)[NPASS]) {
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
      const int row = min(k * RP + ((int)threadIdx.x >> gsh), MB - 1);
      const int off = ((mbase + row) * a.ssq_ld + ((int)threadIdx.x & (G - 1)) * 4) * 4;
      dst[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, 0));
    }
  };
  if constexpr (NORM) load_norm(m_base, sv);
  // 4. epilogue inputs that do not depend on the product
  float2 pcs = make_float2(0.f, 0.f);
  int pslot = 0;
  float ph[2] = {0.f, 0.f}, pg = 0.f;
  auto load_epi = [&](int mbase) {
    if constexpr (EPI == EPI_QKV) {   // NT == 1: rotary pairs 8jj..8jj+7 of this tile's head
      const int half = a.head_dim / 2, jj = tg % (a.head_dim / 16);
      const int m = min(mbase + min((int)threadIdx.x / 8, MB - 1), m_last);
      pcs = a.row_cs[(size_t)m * half + 8 * jj + threadIdx.x % 8];
      pslot = a.row_slot[min(mbase + min((int)threadIdx.x, MB - 1), m_last)];
    }
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int e = min((int)threadIdx.x + b * NTH, NT * MB * 16 - 1);
        const int t = e / (MB * 16), r = (e / 16) % MB, n = e % 16;
        ph[b] = a.h[(size_t)min(mbase + r, m_last) * a.hidden + (tg * NT + t) * 16 + n];
      }
      pg = a.gain_next[tg * NT * 16 + min((int)threadIdx.x, NT * 16 - 1)];
    }
  };
  load_epi(m_base);

  // ---- stores to LDS: the slab and the epilogue inputs of row block m_base ----
  auto stage = [&]() {
    if constexpr (!DIRECT) {
#pragma unroll
      for (int b = 0; b < SBX; ++b) {
        const int e = threadIdx.x + b * NTH;
        if (e < total) *reinterpret_cast<uint4*>(slab + (e >> fsh) * XSTR + (e & (FPR - 1)) * 16) = xs[b];
      }
      for (int e = threadIdx.x + SBX * NTH; e < total; e += NTH) {   // K ranges above SBX*NTH fragments
        const int r = e >> fsh, q = e & (FPR - 1);
        *reinterpret_cast<uint4*>(slab + r * XSTR + q * 16) =
            m_base + r < m_end ? *reinterpret_cast<const uint4*>(xb + (size_t)(m_base + r) * a.ldx + q * PER)
                                 : make_uint4(0, 0, 0, 0);
      }
    }
    if constexpr (EPI == EPI_QKV) {
      float2* s_cs = reinterpret_cast<float2*>(smem + L.pre);
      int* s_slot = reinterpret_cast<int*>(smem + L.pre + MB * 8 * 8);
      if (threadIdx.x < MB * 8) s_cs[threadIdx.x] = pcs;
      if (threadIdx.x < MB) s_slot[threadIdx.x] = pslot;
    }
    if constexpr (EPI == EPI_RESID) {
      float* s_h = reinterpret_cast<float*>(smem + L.pre);
      float* s_g = s_h + NT * MB * 16;
#pragma unroll
      for (int b = 0; b < 2; ++b)
        if (threadIdx.x + b * NTH < NT * MB * 16) s_h[threadIdx.x + b * NTH] = ph[b];
      if (threadIdx.x < NT * 16) s_g[threadIdx.x] = pg;
    }
  };
  if constexpr (!MLOOP) {
    stage();
    // (DIRECT: the staged epilogue inputs are read only after the slice reduction's barrier)
    if constexpr (!DIRECT) __syncthreads();
  }

  // The LM head's single-block workgroups stage the slab and 1/rms once, then walk their tile
  // groups (stride gridDim.x), loading the next group's weights while the current one is
  // multiplied and reduced.  The looped form stages each row block in turn.  Every other GEMM
  // runs the body once.
  const int n_groups = a.n_tiles / NT;
  bool first = true;
  float4 svn[NPASS];
  for (;;) {
  int tg_next = tg + (int)gridDim.x;
  bool more = LOOP && tg_next < n_groups;
  uint4 wn[KPW];
  if constexpr (LOOP) {
    // branch-free: past the last group, the current group's lines are read again (L2 hits)
    const int tg_load = more ? tg_next : tg;
    const uint4* wp = a.W + ((size_t)(tg_load * NT + tsub) * ksteps + kstep0) * kWave + lane;
#pragma unroll
    for (int s = 0; s < KPW; ++s) wn[s] = wp[(size_t)s * kWave];
  }
  int mb_next = mb;
  if constexpr (MLOOP) {
    stage();
    __syncthreads();
    // branch-free: after the last row block, the current block's lines are read again (L2 hits)
    mb_next = mb + (int)gridDim.z;
    more = mb_next < m_blocks;
    const int mb_load = more ? mb_next : mb;
    load_slab(mb_load * MB);
    if constexpr (NORM) load_norm(mb_load * MB, svn);
    load_epi(mb_load * MB);
  }
  // 5. MFMA chain over this wave's K steps
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (cwave) {
    if constexpr (DIRECT) {
#pragma unroll
      for (int s = 0; s < KPW; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma_wa(acc[mt], wf[s], bx[s][mt], T());
    } else {
      // activation fragments of step s + 1 are read from LDS while step s multiplies (a read
      // awaited right before each product would expose the LDS latency on every step)
      auto bfrag = [&](int s, int mt) {
        const int kb = ((ksl * KPW + s) * KS + PER * (lane / 16)) * (int)sizeof(T);
        return *reinterpret_cast<const uint4*>(slab + (mt * 16 + lane % 16) * XSTR + kb);
      };
      uint4 bc[MT], bn[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) bc[mt] = bfrag(0, mt);
#pragma unroll
      for (int s = 0; s < KPW; ++s) {
        if (s + 1 < KPW) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) bn[mt] = bfrag(s + 1, mt);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of this step's products
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma_wa(acc[mt], wf[s], bc[mt], T());
        if (s + 1 < KPW) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) bc[mt] = bn[mt];
        }
      }
    }
  }
  if (NORM && (first || MLOOP)) {
    // 1/rms of each row (needed only by the epilogue, so it runs behind the MFMA chain): each
    // lane adds its 4 partials in column order, then a fixed butterfly over the row's G lanes
    // hidden is a power of two, so the product with its reciprocal is the quotient exactly; passes
    // past the block's rows are skipped
    const float rh = 1.0f / (float)a.hidden;
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
      if (k * RP >= MB) break;
      const float sum = lane_group_sum(((sv[k].x + sv[k].y) + sv[k].z) + sv[k].w, G);
      const int row = k * RP + ((int)threadIdx.x >> gsh);
      if (((int)threadIdx.x & (G - 1)) == 0 && row < MB) s_inv[row] = 1.0f / sqrtf(sum * rh + a.eps);
    }
  }
  // 6. K-slice partial tiles added in slice order: element i of lane l of a tile is
  //    [4(l/16) + i][l % 16] of the transposed product, i.e. row 16mt + l%16, column 4(l/16) + i
  if (cwave) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * kWave + lane] = acc[mt];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NT * MT * kWave; e += NTH) {
    const int t = e / (MT * kWave), mt = (e / kWave) % MT, l = e % kWave;
    f32x4_t v = red[((t * KSL) * MT + mt) * kWave + l];
    for (int j = 1; j < KSL; ++j) v = v + red[((t * KSL + j) * MT + mt) * kWave + l];
    float* dst = ctile + (t * MB + mt * 16 + l % 16) * 17 + 4 * (l / 16);
    if constexpr (EPI == EPI_LOGITS) {
      // the logits z = product * 1/rms of the row, scaled here rather than in a pass of their own
      const int r = mt * 16 + l % 16, m = m_base + r;
      const float inv = s_inv[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = v[i] * inv;
        dst[i] = z;
        const int col = (tg * NT + t) * 16 + 4 * (l / 16) + i;
        if (a.logits && m < m_end && col < a.vocab) a.logits[(size_t)m * a.vocab + col] = z;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = v[i];
    }
  }
  __syncthreads();

  // 7. epilogue
  if constexpr (EPI == EPI_QKV) {
    const float2* s_cs = reinterpret_cast<const float2*>(smem + L.pre);
    const int* s_slot = reinterpret_cast<const int*>(smem + L.pre + MB * 8 * 8);
    const int hd = a.head_dim, half = hd / 2, tph = hd / 16;
    const int hh = tg / tph, jj = tg % tph;
    const int kind = hh < a.n_heads ? 0 : (hh < a.n_heads + a.n_kv ? 1 : 2);   // q, k, v
    const int head = kind == 0 ? hh : (kind == 1 ? hh - a.n_heads : hh - a.n_heads - a.n_kv);
    for (int e = threadIdx.x; e < MB * 8; e += NTH) {
      const int r = e / 8, c = e % 8;
      const int m = m_base + r;
      if (m >= m_end) continue;
      const float inv = s_inv[r];
      const float* ct = ctile + r * 17;
      float x1 = ct[c] * inv, x2 = ct[c + 8] * inv;
      const int i = 8 * jj + c;                 // rotary pair (i, i + hd/2)
      if (kind != 2) {
        const float2 cs = s_cs[e];
        const float o1 = x1 * cs.x - x2 * cs.y;
        const float o2 = x2 * cs.x + x1 * cs.y;
        x1 = o1; x2 = o2;
      }
      if (kind == 0) {
        T* dst = reinterpret_cast<T*>(a.q) + (size_t)m * a.q_ld + head * hd;
        dst[i] = Act<T>::from_f(x1);
        dst[i + half] = Act<T>::from_f(x2);
      } else {
        const int sl = s_slot[r];
        T* pool = reinterpret_cast<T*>(a.kv_pool);
        pool[kv_off(a.layer, a.n_pages, sl / kPage, kind - 1, a.n_kv, head, sl % kPage, i, hd)] = Act<T>::from_f(x1);
        pool[kv_off(a.layer, a.n_pages, sl / kPage, kind - 1, a.n_kv, head, sl % kPage, i + half, hd)] =
            Act<T>::from_f(x2);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    resid_epilogue<T, MB>(a, ctile, reinterpret_cast<const float*>(smem + L.pre), tg, NT, m_base, m_end);
  } else if constexpr (EPI == EPI_PARTIAL) {
    for (int e = threadIdx.x; e < NT * MB * 16; e += NTH) {
      const int t = e / (MB * 16), r = (e / 16) % MB, n = e % 16;
      const int m = m_base + r;
      if (m >= m_end) continue;
      const int col = (tg * NT + t) * 16 + n;
      a.part[((size_t)split * a.M + m) * a.part_ld + col] = ctile[(t * MB + r) * 17 + n];
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int e = threadIdx.x; e < NT * MB * 8; e += NTH) {
      const int t = e / (MB * 8), r = (e / 8) % MB, c = e % 8;
      const int m = m_base + r;
      if (m >= m_end) continue;
      const float* ct = ctile + (t * MB + r) * 17;
      const float g = ct[c] * s_inv[r];
      const float u = ct[c + 8] * s_inv[r];
      reinterpret_cast<T*>(a.act)[(size_t)m * a.act_ld + (tg * NT + t) * 8 + c] = Act<T>::from_f(silu_f(g) * u);
    }
  } else {  // EPI_LOGITS (the reduction above left the scaled logits z in ctile)
    // one (top1, id, top2) record per row over the workgroup's NT*16 columns: 8 lanes per row
    // scan 2*NT columns each in column order (all reads first, then a branch-free scan), then
    // merge across the 8 lanes by DPP moves
    constexpr int kMaxCpl = 8;                        // 2 * NT columns per lane, NT <= 4
    const int cpl = 2 * NT;
    const int groups = NTH / 8;
    const int n_it = (MB + groups - 1) / groups;
    for (int it = 0; it < n_it; ++it) {
      const int r = it * groups + threadIdx.x / 8, sub = threadIdx.x % 8;
      const int rr = min(r, MB - 1);
      float zv[kMaxCpl];
#pragma unroll
      for (int k = 0; k < kMaxCpl; ++k) {
        const int cc = sub * cpl + min(k, cpl - 1);   // column within the workgroup's span
        zv[k] = ctile[((cc / 16) * MB + rr) * 17 + cc % 16];
      }
      Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
      bool nan = false;
#pragma unroll
      for (int k = 0; k < kMaxCpl; ++k) {
        const int col = tg * NT * 16 + sub * cpl + k;
        const float z = zv[k];
        // the sequential update (a new maximum pushes the old one to second place; equal values
        // keep the earlier, lower column) as selects
        const bool ok = k < cpl && r < MB && col < a.vocab && col != a.mask_id;
        const bool isnan = ok && z != z;
        const bool gt1 = ok && !isnan && z > best.v1;
        const bool gt2 = ok && !isnan && !gt1 && z > best.v2;
        best.v2 = gt1 ? best.v1 : (gt2 ? z : best.v2);
        best.v1 = gt1 ? z : best.v1;
        best.i1 = gt1 ? col : best.i1;
        nan = nan || isnan;
      }
      if (nan) best = Top2{NAN, -1, NAN};
      best = merge_top2(best, dpp_top2<0xB1>(best));    // quad_perm [1,0,3,2]
      best = merge_top2(best, dpp_top2<0x4E>(best));    // quad_perm [2,3,0,1]
      best = merge_top2(best, dpp_top2<0x141>(best));   // row_half_mirror
      const int m = m_base + r;
      if (sub == 0 && r < MB && m < m_end) {
        const size_t o = (size_t)m * a.am_ld + tg;
        a.am_v1[o] = best.v1;
        a.am_i1[o] = best.i1;
        a.am_v2[o] = best.v2;
      }
      if (a.am_s) {
        // softmax denominator of the group relative to its own max (the confidence of the
        // direct-diffusion step); the same 8 lanes, the same columns, a fixed lane order
        float se = 0.f;
        if (r < MB && best.i1 >= 0 && best.v1 > -INFINITY) {
          for (int k = 0; k < cpl; ++k) {
            const int cc = sub * cpl + k;
            const int col = tg * NT * 16 + cc;
            if (col >= a.vocab || col == a.mask_id) continue;
            se += __builtin_amdgcn_exp2f((ctile[((cc / 16) * MB + r) * 17 + cc % 16] - best.v1) * a.am_scale);
          }
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) se += __shfl_xor(se, o);
        if (sub == 0 && r < MB && m < m_end) a.am_s[(size_t)m * a.am_ld + tg] = best.i1 >= 0 ? se : NAN;
      }
    }
  }
  if (!more) break;
  if constexpr (LOOP) {
    tg = tg_next;
#pragma unroll
    for (int s = 0; s < KPW; ++s) wf[s] = wn[s];
  }
  if constexpr (MLOOP) {
    mb = mb_next;
    m_base = mb * MB;
    m_end = min(a.M, m_base + MB);
#pragma unroll
    for (int k = 0; k < NPASS; ++k) sv[k] = svn[k];
  }
  first = false;
  __syncthreads();   // red, ctile, the slab and the staged inputs are reused by the next item
  }
  stamp_end(a.stamp);
}

// ---------------------------------------------------------------------------
// Fused tail of one decoder layer for decode forwards of at most 48 rows: O + residual, gate|up
// + SwiGLU and down + residual in one kernel of kTailWgs workgroups (one per CU), separated by
// two grid barriers.  Each workgroup issues the loads of its next weight slice well before the
// barrier that precedes its use (gate|up: 64 KB behind the O products, down: 128 KB behind the
// gate|up activations), so those weights stream in from HBM while the current stage and the
// barrier run, instead of each GEMM starting cold after a kernel boundary.  The data that crosses a barrier inside the kernel (the residual h, the next
// GEMM input xg and the norm partials from O; the SwiGLU output from gate|up) is written and read
// device-coherently (write-through stores, sc1 loads), so the barrier needs no cache flush.
//
// Each stage performs, for every row, exactly the operations of k_gemm with the same plan (O and
// down: one 16-column tile, 8 K slices; gate|up: 2 tiles, 4 K slices; slice partial tiles added
// in slice order, the same 1/rms butterfly and epilogues, no contraction), so rows stay
// bit-identical to the unfused kernels whatever kernel computes them.  Waves 0-7 own the K slices
// as in k_gemm.  A wave's memory operations complete in issue order, and issuing a load can stall
// the wave while the CU's memory queue is full, so every load is placed by what it must not delay:
// the gate|up weights go out once the O stage's products are done, the down weights once the
// gate|up activations are in.  A ninth wave (kStoreWave) makes every
// store that crosses a barrier and loads nothing, so it alone waits for its stores before the
// workgroup arrives, and the other waves keep their weight loads in flight across the barriers.
//
// Barriers: arrivals count on 8 partition counters (workgroup w in partition w % 8); the arrival
// that completes a partition writes that partition's done flag, and every workgroup polls the 8
// done flags (one lane each).  No polled word is the target of an atomic: 256 pollers on the word
// that arrivals add to delay the adds.  (Measured per round at n = 1280: partition leaders adding
// to a global counter that everyone polls, 1778 us; the same with the completing arrival writing
// release flags, 1743 us; everyone polling the 8 partition counters themselves, 1888 us; done
// flags, 1715 us.)  Counters and flags grow monotonically: a launch reads the generation word at
// entry and waits for (generation + 1); workgroup 0 advances the generation once it has passed the
// second barrier, by which time every workgroup has read it.  Waits are bounded: past kSpinMax
// polls a workgroup sets *err and leaves (results are then invalid, and the argmax and accept
// kernels report it).
// ---------------------------------------------------------------------------
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
constexpr int kTailParts = 8;
constexpr int kSpinMax = 1 << 16;
constexpr int kStoreWave = kGemmThreads / kWave;        // the ninth wave
constexpr int kTailThreads = kGemmThreads + kWave;

// Arrival and polling are the store wave's: it holds no load that could delay its atomic (a wave's
// memory operations complete in issue order, and the other waves have weight loads in flight), and
// no other wave has a store in flight.  Returns whether every workgroup arrived.
__device__ __forceinline__ bool tail_barrier(unsigned long long* sync, int b, unsigned long long gen, int* err,
                                             int* s_flag) {
  if ((int)threadIdx.x / kWave == kStoreWave) {
    const int lane = threadIdx.x % kWave;
    __builtin_amdgcn_s_waitcnt(0);   // this workgroup's coherent stores have completed
    const int p = blockIdx.x % kTailParts;
    const unsigned long long per = kTailWgs / kTailParts;
    unsigned long long* pc = sync + 16 * (1 + 16 * b + p);       // partition counters of barrier b
    unsigned long long* done = sync + 16 * (9 + 16 * b);          // its done flags, one per partition
    if (lane == 0) {
      const unsigned long long old = __hip_atomic_fetch_add(pc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == (gen + 1) * per) st_coh(done + 16 * p, gen + 1);
    }
    // lanes 0-7 each wait for one partition; a lane whose partition is done stops loading
    bool ok = lane >= kTailParts;
    int spins = 0;
    for (;;) {
      if (!ok) ok = ld_coh(done + 16 * (lane % kTailParts)) >= gen + 1;
      if (__all(ok) || ++spins >= kSpinMax) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) {
      const bool passed = spins < kSpinMax;
      if (!passed) st_coh(err, 1);
      s_flag[0] = passed;
    }
  }
  __syncthreads();
  return s_flag[0] != 0;
}

template <int KPW_O, int KPW_G, int KPW_D>
__global__ __launch_bounds__(kTailThreads) void k_layer_tail(TailArgs ta) {
#pragma clang fp contract(off)
  using T = bf16_t;
  constexpr int KS = Ty<T>::kStepK, PER = Ty<T>::kPerFrag, NTH = kGemmThreads;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float s_inv[48];
  __shared__ uint32_t s_act[2 * 48 * 4];   // SwiGLU outputs, packed pairs [tile][row][pair]
  __shared__ __align__(16) float s_v[256];  // O stage: residual sums [16 rows][16 columns]
  __shared__ int s_flag[1];
  __shared__ unsigned long long s_gen;
  stamp_begin(ta.stamp);
  const GemmArgs& ao = ta.o;
  const GemmArgs& ag = ta.gu;
  const GemmArgs& ad = ta.d;
  const int w = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool cw = wave < kStoreWave;                 // waves 0-7: the K slices
  const int M = ao.M, m_last = M - 1;
  if ((int)threadIdx.x == kStoreWave * kWave) s_gen = ld_coh(ta.sync);

  // ---- O stage item (k_gemm's DIRECT form: balanced 16-row blocks); its loads first ----
  const int nrb = (M + 15) / 16;
  const int rpb_o = min(16, (M + nrb - 1) / nrb);
  const bool has_o = w < ao.n_tiles * nrb;
  const int to = w % ao.n_tiles, mb_o = w / ao.n_tiles;
  const int mbase_o = mb_o * rpb_o, mend_o = min(M, mbase_o + rpb_o);
  const bool has_d = w < ad.n_tiles * nrb;
  const int td = w % ad.n_tiles, mb_d = w / ad.n_tiles;
  uint4 wo[KPW_O], bxo[KPW_O], wgf[KPW_G], wdf[KPW_D];
  float pho = 0.f, pgo = 0.f;
  // The gate|up weights go out once the O stage's own operands are in (workgroups without an O item:
  // at entry).  Issuing a load can stall the wave until the CU's memory queue takes it, so 64 KB of
  // gate|up weights issued at entry held back the O products behind them (round 1710 -> 1688 us
  // with them issued after the products); they still land well before the first barrier ends.
  auto issue_gu = [&]() {
    asm volatile("" ::: "memory");
    const uint4* gp = ag.W + ((size_t)(w * 2 + wave / 4) * (ag.K / KS) + (wave % 4) * KPW_G) * kWave + lane;
#pragma unroll
    for (int s = 0; s < KPW_G; ++s) wgf[s] = gp[(size_t)s * kWave];
  };
  if (cw) {
    if (has_o) {
      const uint4* wp = ao.W + ((size_t)to * (ao.K / KS) + wave * KPW_O) * kWave + lane;
#pragma unroll
      for (int s = 0; s < KPW_O; ++s) wo[s] = wp[(size_t)s * kWave];
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ao.x), (short)0,
                                                                          mend_o * ao.ldx * (int)sizeof(T), kBufWord3);
#pragma unroll
      for (int s = 0; s < KPW_O; ++s) {
        const int off = ((mbase_o + lane % 16) * ao.ldx + (wave * KPW_O + s) * KS + PER * (lane / 16)) * (int)sizeof(T);
        bxo[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
      }
      const int e = min((int)threadIdx.x, 255), r = (e / 16) % 16, n = e % 16;
      pho = ao.h[(size_t)min(mbase_o + r, m_last) * ao.hidden + to * 16 + n];
      pgo = ao.gain_next[to * 16 + min((int)threadIdx.x, 15)];
    }
    if (!has_o) issue_gu();
  }
  __syncthreads();
  const unsigned long long gen = s_gen;

  // ---- stage 1: O + residual (h, xg, norm partials written coherently by the store wave) ----
  if (has_o) {
    const GemmLds L = gemm_lds(1, 8 * KPW_O * KS * (int)sizeof(T), 1, 8, ao.n_ssq, EPI_RESID);
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + L.red);
    float* ctile = reinterpret_cast<float*>(smem + L.ctile);
    float* s_h = reinterpret_cast<float*>(smem + L.pre);
    if (cw) {
      if (threadIdx.x < 256) s_h[threadIdx.x] = pho;
      if (threadIdx.x < 16) s_h[256 + threadIdx.x] = pgo;
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KPW_O; ++s) mma_wa(acc, wo[s], bxo[s], T());
      red[wave * kWave + lane] = acc;
      issue_gu();
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int l = threadIdx.x;
      f32x4_t v = red[l];
      for (int j = 1; j < 8; ++j) v = v + red[j * kWave + l];
      float* dst = ctile + (l % 16) * 17 + 4 * (l / 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = v[i];
    }
    __syncthreads();
    // k_gemm's residual epilogue (v = h + tile, xg = v * gain, each row's 16 squares in order),
    // computed by all waves into LDS; the store wave then writes h as 16-byte pieces, xg as packed
    // pairs and the row sums, coherently
    uint32_t* s_x = s_act;                                  // [16 rows][8 pairs]
    float* s_q = reinterpret_cast<float*>(s_act + 128);     // [16 rows]
    if (threadIdx.x < 256) s_v[threadIdx.x] = s_h[threadIdx.x] + ctile[(threadIdx.x / 16) * 17 + threadIdx.x % 16];
    __syncthreads();
    if (threadIdx.x < 128) {
      const int r = threadIdx.x / 8, c = 2 * (threadIdx.x % 8);
      s_x[threadIdx.x] = (uint32_t)Act<T>::from_f(s_v[r * 16 + c] * s_h[256 + c]) |
                         ((uint32_t)Act<T>::from_f(s_v[r * 16 + c + 1] * s_h[256 + c + 1]) << 16);
    } else if (threadIdx.x < 144) {
      const int r = threadIdx.x - 128;
      float sum = 0.f;
      for (int n = 0; n < 16; ++n) {
        const float v = s_v[r * 16 + n];
        sum += v * v;
      }
      s_q[r] = sum;
    }
    __syncthreads();
    if (wave == kStoreWave) {
      const int nr = mend_o - mbase_o;
      const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(ao.h, (short)0, M * ao.hidden * 4, kBufWord3);
      {
        const int r = lane / 4, q = lane % 4;
        if (r < nr)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4v, *reinterpret_cast<const float4*>(s_v + r * 16 + 4 * q)), hr,
              ((mbase_o + r) * ao.hidden + to * 16 + 4 * q) * 4, 0, kCoh);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = lane + k * kWave, r = e / 8;
        if (r < nr)
          st_coh(reinterpret_cast<uint32_t*>(reinterpret_cast<T*>(ao.xg_out) + (size_t)(mbase_o + r) * ao.hidden +
                                             to * 16) + e % 8, s_x[e]);
      }
      if (lane < nr) st_coh(ao.ssq_out + (size_t)(mbase_o + lane) * ao.ssq_ld + to, s_q[lane]);
    }
  }
  if (!tail_barrier(ta.sync, 0, gen, ta.err, s_flag)) return;

  // ---- stage 2: gate|up + SwiGLU over all rows (one 48-row block; SwiGLU output coherent) ----
  {
    constexpr int MT = 3, MB = 48, KR = 4 * KPW_G * KS, XSTR = KR * (int)sizeof(T) + 16;
    constexpr int FPR = KR / PER, TOTAL = MB * FPR, SB = 12;
    static_assert(TOTAL == SB * NTH, "the gate|up slab is 12 fragments per thread");
    constexpr int fsh = __builtin_ctz(FPR);
    const GemmLds L = gemm_lds(MT, KR * (int)sizeof(T), 2, 4, ag.n_ssq, EPI_SWIGLU);
    unsigned char* slab = smem;
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + L.red);
    constexpr int NPASS = 3;
    const int G = ag.n_ssq / 4, gsh = 31 - __builtin_clz(G), RP = NTH >> gsh;
    float4 sv[NPASS];
    if (cw) {
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ag.x), (short)0,
                                                                          M * ag.ldx * (int)sizeof(T), kBufWord3);
      uint4 xs[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int e = threadIdx.x + b * NTH;
        const int off = ((e >> fsh) * ag.ldx + (e & (FPR - 1)) * PER) * (int)sizeof(T);
        xs[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, kCoh));
      }
      const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ag.ssq), (short)0,
                                                                          M * ag.ssq_ld * 4, kBufWord3);
#pragma unroll
      for (int k = 0; k < NPASS; ++k) {
        const int row = min(k * RP + ((int)threadIdx.x >> gsh), MB - 1);
        const int off = (row * ag.ssq_ld + ((int)threadIdx.x & (G - 1)) * 4) * 4;
        sv[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, kCoh));
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int e = threadIdx.x + b * NTH;
        *reinterpret_cast<uint4*>(slab + (e >> fsh) * XSTR + (e & (FPR - 1)) * 16) = xs[b];
      }
      asm volatile("" ::: "memory");   // the down weights go out once the activations are in
      if (has_d) {
        const uint4* dp = ad.W + ((size_t)td * (ad.K / KS) + wave * KPW_D) * kWave + lane;
#pragma unroll
        for (int s = 0; s < KPW_D; ++s) wdf[s] = dp[(size_t)s * kWave];
      }
    }
    __syncthreads();
    if (cw) {
      const int ksl = wave % 4;
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KPW_G; ++s) {
        const int kb = ((ksl * KPW_G + s) * KS + PER * (lane / 16)) * (int)sizeof(T);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          mma_wa(acc[mt], wgf[s], *reinterpret_cast<const uint4*>(slab + (mt * 16 + lane % 16) * XSTR + kb), T());
      }
      const float rh = 1.0f / (float)ag.hidden;
#pragma unroll
      for (int k = 0; k < NPASS; ++k) {
        if (k * RP >= MB) break;
        const float sum = lane_group_sum(((sv[k].x + sv[k].y) + sv[k].z) + sv[k].w, G);
        const int row = k * RP + ((int)threadIdx.x >> gsh);
        if (((int)threadIdx.x & (G - 1)) == 0 && row < MB) s_inv[row] = 1.0f / sqrtf(sum * rh + ag.eps);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * kWave + lane] = acc[mt];
    }
    __syncthreads();
    // The K-slice reduction and SwiGLU in one pass: thread (t, mt, row lane rl, q) adds, in slice
    // order, the 4 partials of gate columns 4q .. 4q+3 and of up columns 8+4q .. 8+4q+3 of row
    // 16mt + rl (lanes rl + 16q and rl + 16(q+2) of the partial tiles), scales them by 1/rms and
    // forms two packed pairs of SwiGLU outputs (an exponential and a division each) into LDS; the
    // store wave then writes them coherently
    for (int e = threadIdx.x; e < 2 * MT * 32; e += kTailThreads) {
      const int t = e / (MT * 32), mt = (e / 32) % MT, q = (e / 16) % 2, rl = e % 16;
      const int lg = rl + 16 * q, lu = rl + 16 * (q + 2);
      f32x4_t vg = red[((t * 4) * MT + mt) * kWave + lg], vu = red[((t * 4) * MT + mt) * kWave + lu];
      for (int j = 1; j < 4; ++j) {
        vg = vg + red[((t * 4 + j) * MT + mt) * kWave + lg];
        vu = vu + red[((t * 4 + j) * MT + mt) * kWave + lu];
      }
      const int r = mt * 16 + rl;
      const float inv = s_inv[r];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float g0 = vg[2 * p] * inv, u0 = vu[2 * p] * inv;
        const float g1 = vg[2 * p + 1] * inv, u1 = vu[2 * p + 1] * inv;
        s_act[(t * MB + r) * 4 + 2 * q + p] =
            (uint32_t)Act<T>::from_f(silu_f(g0) * u0) | ((uint32_t)Act<T>::from_f(silu_f(g1) * u1) << 16);
      }
    }
    __syncthreads();
    for (int e = lane; wave == kStoreWave && e < 2 * MB * 4; e += kWave) {
      const int t = e / (MB * 4), r = (e / 4) % MB;
      if (r >= M) continue;
      st_coh(reinterpret_cast<uint32_t*>(reinterpret_cast<T*>(ag.act) + (size_t)r * ag.act_ld + (w * 2 + t) * 8) + e % 4,
             s_act[e]);
    }
  }
  if (!tail_barrier(ta.sync, 1, gen, ta.err, s_flag)) return;

  // ---- stage 3: down + residual (16-row blocks; its outputs feed the next kernel) ----
  if (has_d) {
    constexpr int MB = 16, KR = 8 * KPW_D * KS, XSTR = KR * (int)sizeof(T) + 16;
    constexpr int FPR = KR / PER, TOTAL = MB * FPR, SB = 16;
    static_assert(TOTAL == SB * NTH, "the down slab is 16 fragments per thread");
    constexpr int fsh = __builtin_ctz(FPR);
    const GemmLds L = gemm_lds(1, KR * (int)sizeof(T), 1, 8, ad.n_ssq, EPI_RESID);
    unsigned char* slab = smem;
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + L.red);
    float* ctile = reinterpret_cast<float*>(smem + L.ctile);
    float* s_h = reinterpret_cast<float*>(smem + L.pre);
    const int m_base = mb_d * MB, m_end = min(M, m_base + MB);
    if (cw) {
      const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ad.x), (short)0,
                                                                          M * ad.ldx * (int)sizeof(T), kBufWord3);
      uint4 xs[SB];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int e = threadIdx.x + b * NTH;
        const int off = ((m_base + (e >> fsh)) * ad.ldx + (e & (FPR - 1)) * PER) * (int)sizeof(T);
        xs[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, kCoh));
      }
      const int e0 = min((int)threadIdx.x, 255), r0 = (e0 / 16) % 16, n0 = e0 % 16;
      const float ph = ld_coh(ad.h + (size_t)min(m_base + r0, m_last) * ad.hidden + td * 16 + n0);
      const float pg = ad.gain_next[td * 16 + min((int)threadIdx.x, 15)];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int e = threadIdx.x + b * NTH;
        *reinterpret_cast<uint4*>(slab + (e >> fsh) * XSTR + (e & (FPR - 1)) * 16) = xs[b];
      }
      if (threadIdx.x < 256) s_h[threadIdx.x] = ph;
      if (threadIdx.x < 16) s_h[256 + threadIdx.x] = pg;
    }
    __syncthreads();
    if (cw) {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KPW_D; ++s) {
        const int kb = ((wave * KPW_D + s) * KS + PER * (lane / 16)) * (int)sizeof(T);
        mma_wa(acc, wdf[s], *reinterpret_cast<const uint4*>(slab + (lane % 16) * XSTR + kb), T());
      }
      red[wave * kWave + lane] = acc;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int l = threadIdx.x;
      f32x4_t v = red[l];
      for (int j = 1; j < 8; ++j) v = v + red[j * kWave + l];
      float* dst = ctile + (l % 16) * 17 + 4 * (l / 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = v[i];
    }
    __syncthreads();
    resid_epilogue<T, 16, false>(ad, ctile, s_h, td, 1, m_base, m_end);
  }
  // every workgroup has read the generation word (each arrived at the second barrier after reading
  // it): the next launch may use the next one
  if (w == 0 && (int)threadIdx.x == kStoreWave * kWave) st_coh(ta.sync, gen + 1);
  stamp_end(ta.stamp);
}

// ---------------------------------------------------------------------------
// Large-M GEMM for prefill and teacher-forced forwards (M >= 128 rows, bf16):
// the same packed weight fragments and fused epilogues as k_gemm (QKV + RoPE +
// KV write, residual + next norm input, SwiGLU), tiled for operand reuse.  A
// workgroup of 4 waves (2 x 2) owns a (32 RT) x (32 CT) output block and walks
// the whole K range in 32-wide steps.  Each step's fragments (2CT weight
// fragments of 1 KiB, 2RT activation fragments of 1 KiB in MFMA operand
// layout) go straight from global memory to LDS (16 B per lane), NS steps in
// flight, one barrier per step; each wave multiplies its RT x CT 16x16 tiles
// from LDS.  Forwards without decode rows (prefill, teacher forcing) use it as
// is.  EXACT: the per-element arithmetic of k_gemm, for tall decode forwards
// (batched rounds): each K slice of k_gemm's plan (a.KSL slices of
// ksteps/a.KSL steps) gets its own MFMA chain from zero and the slices are
// added in order; 1/rms, RoPE, SwiGLU and the residual sums of squares follow
// k_gemm's operation order; no multiply-add contraction.  A row's results are
// then bit-identical to k_gemm's, whatever the row count or tile shape.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt immediate: vmcnt[3:0] and [15:14]; expcnt and lgkmcnt left at "no wait"
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane (lds_base is
// wave-uniform; it goes through M0).  Issued as inline assembly so the compiler does not pair
// every later LDS read with a wait for all outstanding loads; the caller waits with wait_vmcnt
// and a barrier before reading the destination.  The compiler does not preserve M0 across inline
// assembly; in the built k_gemm_big kernels every M0 write and read is this block's own.
__device__ __forceinline__ void load_lds16(const void* gptr, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

// JIT (the wide non-exact blocks): the fragments of a step are read from LDS as the products use
// them, with no register copy of the next step, so that the kernel fits two workgroups per CU;
// each covers the other's LDS latency.  The copy of step s + NS - 1 then goes into the buffer of
// step s - 1, which every wave has finished reading at step s's barrier.
template <int RT, int CT, bool EXACT, int WC>
constexpr bool big_jit() { return !EXACT && RT * CT * WC >= 64; }

// Waves as 2 x WC, each RT row tiles x CT column tiles: a block of 32 RT rows x 16 WC CT columns.
// WC = 4 (eight waves, two workgroups per CU: four waves per SIMD) for the widest non-exact GEMM:
// one wave per SIMD left every LDS, matrix-core and barrier latency of a step exposed.
template <int EPI, int RT, int CT, int NS, bool EXACT, int WC = 2>
__global__ __launch_bounds__(2 * WC * kWave, (WC == 4 ? 4 : (big_jit<RT, CT, EXACT, WC>() ? 2 : 1))) void k_gemm_big(GemmArgs a) {
#pragma clang fp contract(off)
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LOGITS);
  static_assert(EPI != EPI_LOGITS || (EXACT && CT == 4 && WC == 2), "LM head: exact form, one 4-tile group per wave");
  static_assert(!EXACT || WC == 2, "the exact form runs four waves");
  constexpr int NW = 2 * WC;               // waves
  constexpr int NF = WC * CT + 2 * RT;     // 1 KiB fragments per step: weights first, then activations
  constexpr int FPW = NF / NW;             // fragments each wave stages per step
  constexpr int BM = 32 * RT;
  static_assert(NF % NW == 0 && NS >= 2, "tile shape");
  extern __shared__ __align__(16) unsigned char smem[];   // [NS][NF][1 KiB], then 1/rms [BM]
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wr = wave / WC, wc = wave % WC;
  const int tn0 = blockIdx.x * WC * CT;    // first 16-column tile of the block
  const int m0 = blockIdx.y * BM;          // first row of the block
  const int ksteps = a.K / Ty<bf16_t>::kStepK;
  float* s_inv = reinterpret_cast<float*>(smem + NS * NF * 1024);
  const unsigned lds0 = (unsigned)(size_t)(lds_ptr_t)smem;   // LDS byte address of the staging area
  stamp_begin(a.stamp);

  // this wave's fragments of a step: f = wave + NW i; weights for f < WC CT, activations after
  const uint4* src[FPW];
  int stride[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = wave + NW * i;
    if (f < WC * CT) {
      src[i] = a.W + (size_t)(tn0 + f) * ksteps * kWave + lane;
      stride[i] = kWave;
    } else if (a.xpk) {
      // fragment-major activations: the (row tile, K step) fragment is 1 KiB in lane order; row
      // tiles past the last one (only in the block's padding) read the last
      const int rt = min(m0 / 16 + (f - WC * CT), (a.M + 15) / 16 - 1);
      src[i] = reinterpret_cast<const uint4*>(a.x) + (size_t)rt * ksteps * kWave + lane;
      stride[i] = kWave;
    } else {
      const int row = min(m0 + 16 * (f - WC * CT) + lane % 16, a.M - 1);   // rows past M: any valid row
      src[i] = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(a.x) + (size_t)row * a.ldx +
                                              (lane / 16) * 8);
      stride[i] = Ty<bf16_t>::kStepK / 8;   // uint4 per 32 K
    }
  }
  auto issue = [&](int s) {
    const int ss = min(s, ksteps - 1);      // steps past the end reload the last one (never read)
    const unsigned buf = lds0 + (s % NS) * NF * 1024;
#pragma unroll
    for (int i = 0; i < FPW; ++i) load_lds16(src[i] + (size_t)ss * stride[i], buf + (wave + NW * i) * 1024);
  };

  if constexpr (NORM && EXACT) {
    // k_gemm's order: G = n_ssq/4 lanes per row each add their 4 partials in column order,
    // then the same fixed butterfly over the row's G lanes
    const int G = a.n_ssq / 4, gsh = 31 - __builtin_clz(G), RP = 256 >> gsh;
    const float rh = 1.0f / (float)a.hidden;   // a power of two: x * rh == x / hidden
    for (int k = 0; k * RP < BM; ++k) {
      const int row = k * RP + ((int)threadIdx.x >> gsh);
      const int m = min(m0 + min(row, BM - 1), a.M - 1);
      const float4 sv = *reinterpret_cast<const float4*>(a.ssq + (size_t)m * a.ssq_ld + ((int)threadIdx.x & (G - 1)) * 4);
      const float sum = lane_group_sum(((sv.x + sv.y) + sv.z) + sv.w, G);
      if (((int)threadIdx.x & (G - 1)) == 0 && row < BM) s_inv[row] = 1.0f / sqrtf(sum * rh + a.eps);
    }
  } else if constexpr (NORM) {
    // 1/rms of the block's rows from the per-16-column sums of squares, two threads per row
    const int r = threadIdx.x / 2, h2 = threadIdx.x % 2;
    float sum = 0.f;
    if (r < BM) {
      const int m = min(m0 + r, a.M - 1);
      const float* sp = a.ssq + (size_t)m * a.ssq_ld + h2 * (a.n_ssq / 2);
      for (int k = 0; k < a.n_ssq / 2; ++k) sum += sp[k];
    }
    sum += __shfl_xor(sum, 1);
    if (r < BM && h2 == 0) s_inv[r] = 1.0f / sqrtf(sum / (float)a.hidden + a.eps);
  }

  // NS steps in flight; step s+1's operands are read from LDS into registers while step s
  // multiplies (register double buffer), one barrier per step.  JIT: NS - 1 steps in flight
  // beside the one being read.
  constexpr bool JIT = big_jit<RT, CT, EXACT, WC>();
#pragma unroll
  for (int s = 0; s < (JIT ? NS - 1 : NS); ++s) issue(s);
  f32x4_t acc[CT][RT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[c][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto rd = [&](int s, uint4* w, uint4* x) {
    const unsigned char* buf = smem + (s % NS) * NF * 1024;
#pragma unroll
    for (int c = 0; c < CT; ++c) w[c] = *reinterpret_cast<const uint4*>(buf + (wc * CT + c) * 1024 + lane * 16);
#pragma unroll
    for (int r = 0; r < RT; ++r) x[r] = *reinterpret_cast<const uint4*>(buf + (WC * CT + wr * RT + r) * 1024 + lane * 16);
  };
  uint4 wf[CT], xf[RT];
  // EXACT: acc holds the current K slice's chain, tot the slices so far (added in slice order)
  f32x4_t tot[CT][RT];
  const int kpw = EXACT ? ksteps / a.KSL : ksteps;
  int left = kpw;
  bool first_slice = true;
  if constexpr (JIT) {
    for (int s = 0; s < ksteps; ++s) {
      wait_vmcnt<FPW * (NS - 2)>();        // step s has landed (steps past the end reload the last)
      __syncthreads();                     // for every wave, and every wave is done with step s - 1
      issue(s + NS - 1);                   // into step s - 1's buffer
      const unsigned char* buf = smem + (s % NS) * NF * 1024;
#pragma unroll
      for (int r = 0; r < RT; ++r) xf[r] = *reinterpret_cast<const uint4*>(buf + (WC * CT + wr * RT + r) * 1024 + lane * 16);
      // a raised wave priority while the products issue (the other waves' loads and LDS reads wait;
      // measured on four-wave blocks: 43.6 -> 42.6 us for the 1088-row gate|up)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const uint4 w = *reinterpret_cast<const uint4*>(buf + (wc * CT + c) * 1024 + lane * 16);
#pragma unroll
        for (int r = 0; r < RT; ++r) mma_wa(acc[c][r], w, xf[r], bf16_t());
      }
      __builtin_amdgcn_s_setprio(0);
    }
  } else {
  wait_vmcnt<FPW * (NS - 1)>();            // step 0 has landed
  __syncthreads();
  rd(0, wf, xf);
  for (int s = 0; s < ksteps; ++s) {
    wait_vmcnt<FPW * (NS - 2)>();          // step s+1 has landed (steps past the end reload the last)
    __syncthreads();                       // and every wave holds step s in registers
    issue(s + NS);                         // into step s's buffer
    uint4 wn[CT], xn[RT];
    rd(s + 1, wn, xn);
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int r = 0; r < RT; ++r) mma_wa(acc[c][r], wf[c], xf[r], bf16_t());
    if constexpr (EXACT) {
      if (--left == 0) {                   // end of a K slice (uniform)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            tot[c][r] = first_slice ? acc[c][r] : tot[c][r] + acc[c][r];
            acc[c][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        first_slice = false;
        left = kpw;
      }
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) wf[c] = wn[c];
#pragma unroll
    for (int r = 0; r < RT; ++r) xf[r] = xn[r];
  }
  }
  wait_vmcnt<0>();
  if constexpr (EXACT) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[c][r] = tot[c][r];
  }

  // epilogue: element i of lane l of tile (c, r) is row 16 r' + l%16, column 16 tg + 4(l/16) + i
  const int q = lane / 16;
  if constexpr (EPI == EPI_LOGITS) {
    // LM head: a wave's 4 tiles are one 64-column group of k_gemm's plan.  Its (top1, id, top2)
    // record per row is a function of the group's values alone (lowest id among equal maxima,
    // second value of the multiset, NaN if any counted value is NaN), so the row's 4 lanes scan
    // their columns in increasing order and merge.
    const int grp = (tn0 + wc * CT) / 4;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rl = 16 * (wr * RT + r) + lane % 16;
      const int m = m0 + rl;
      const float inv = s_inv[rl];
      Top2 best{-INFINITY, 0x7fffffff, -INFINITY};
      bool nan = false;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = (tn0 + wc * CT + c) * 16 + 4 * q + i;
          const float z = acc[c][r][i] * inv;
          if (a.logits && m < a.M && col < a.vocab) a.logits[(size_t)m * a.vocab + col] = z;
          if (col >= a.vocab || col == a.mask_id) continue;
          if (z != z) { nan = true; continue; }
          if (z > best.v1) { best.v2 = best.v1; best.v1 = z; best.i1 = col; }
          else if (z > best.v2) { best.v2 = z; }
        }
      if (nan) best = Top2{NAN, -1, NAN};
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const Top2 other{__shfl_xor(best.v1, o), __shfl_xor(best.i1, o), __shfl_xor(best.v2, o)};
        best = merge_top2(best, other);
      }
      if (q == 0 && m < a.M) {
        const size_t o = (size_t)m * a.am_ld + grp;
        a.am_v1[o] = best.v1;
        a.am_i1[o] = best.i1;
        a.am_v2[o] = best.v2;
      }
    }
    stamp_end(a.stamp);
    return;
  }
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int tg = tn0 + wc * CT + c;
    // QKV: this tile column's rotary factors and KV slots for all RT row tiles, loaded before
    // any is used (loads inside the per-tile branches below were each awaited on the spot)
    const int qq = q & 1;
    int slr[RT];
    float4 csr[RT][2];
    float4 hr[RT], gn;                   // RESID: residual rows and next-norm gains, likewise
    if constexpr (EPI == EPI_RESID) {
      const int n0 = tg * 16 + 4 * q;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int mcr = min(m0 + 16 * (wr * RT + r) + lane % 16, a.M - 1);
        hr[r] = *reinterpret_cast<const float4*>(a.h + (size_t)mcr * a.hidden + n0);
      }
      gn = *reinterpret_cast<const float4*>(a.gain_next + n0);
    }
    if constexpr (EPI == EPI_QKV) {
      const int half = a.head_dim / 2, jj = tg % (a.head_dim / 16);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int mcr = min(m0 + 16 * (wr * RT + r) + lane % 16, a.M - 1);
        slr[r] = a.row_slot[mcr];
        const float4* cp = reinterpret_cast<const float4*>(a.row_cs + (size_t)mcr * half + 8 * jj + 4 * qq);
        csr[r][0] = cp[0];
        csr[r][1] = cp[1];
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int rl = 16 * (wr * RT + r) + lane % 16;     // row within the block
      const int m = m0 + rl;
      const bool ok = m < a.M;
      const int mc = ok ? m : a.M - 1;
      float z[4], zo[4];
      if constexpr (EPI == EPI_QKV) {
        const int hd = a.head_dim, half = hd / 2, tph = hd / 16;
        const int hh = tg / tph, jj = tg % tph;
        const int kind = hh < a.n_heads ? 0 : (hh < a.n_heads + a.n_kv ? 1 : 2);
        const int head = kind == 0 ? hh : (kind == 1 ? hh - a.n_heads : hh - a.n_heads - a.n_kv);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = acc[c][r][i] * s_inv[rl];
#pragma unroll
        for (int i = 0; i < 4; ++i) zo[i] = xor32_get(z[i]);   // the rotary partner column (c +- 8)
        {
          // q row, or the K/V block of the row's slot (dim d at dst[d * dstr])
          bf16_t* dst;
          int dstr = 1;
          if (kind == 0) {
            dst = reinterpret_cast<bf16_t*>(a.q) + (size_t)mc * a.q_ld + head * hd;
          } else {
            const int sl = slr[r];
            dst = reinterpret_cast<bf16_t*>(a.kv_pool) +
                  kv_off(a.layer, a.n_pages, sl / kPage, kind - 1, a.n_kv, head, sl % kPage, 0, hd);
            if (kind == 2) dstr = kPage;
          }
          const float csv[8] = {csr[r][0].x, csr[r][0].y, csr[r][0].z, csr[r][0].w,
                                csr[r][1].x, csr[r][1].y, csr[r][1].z, csr[r][1].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pr = 8 * jj + 4 * qq + i;                      // rotary pair index
            const int dim = (q < 2 ? 0 : half) + pr;
            float o = z[i];
            if (kind != 2) {
              const float cx = csv[2 * i], cy = csv[2 * i + 1];
              o = q < 2 ? z[i] * cx - zo[i] * cy : z[i] * cx + zo[i] * cy;
            }
            if (ok) dst[dim * dstr] = f2h(o);
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = acc[c][r][i] * s_inv[rl];
#pragma unroll
        for (int i = 0; i < 4; ++i) zo[i] = xor32_get(z[i]);
        // lanes l and l ^ 32 hold the gate (columns 4q..) and up (8 + 4(q-2)..) values of the same
        // row and four columns; after the swap each has both, and the pair splits the four outputs
        if (ok) {
          const int hi = q >> 1, qq2 = q & 1;
          const float g0 = hi ? zo[2] : z[0], u0 = hi ? z[2] : zo[0];
          const float g1 = hi ? zo[3] : z[1], u1 = hi ? z[3] : zo[1];
          const uint32_t w2 = (uint32_t)f2h(silu_f(g0) * u0) | ((uint32_t)f2h(silu_f(g1) * u1) << 16);
          const int col = tg * 8 + 4 * qq2 + 2 * hi;
          bf16_t* act = reinterpret_cast<bf16_t*>(a.act);
          *reinterpret_cast<uint32_t*>(act + (a.opk ? pk_off(m, col, a.act_ld) : (size_t)m * a.act_ld + col)) = w2;
        }
      } else {  // EPI_RESID
        const int n0 = tg * 16 + 4 * q;
        const float hv[4] = {hr[r].x, hr[r].y, hr[r].z, hr[r].w};
        const float gv[4] = {gn.x, gn.y, gn.z, gn.w};
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = hv[i] + acc[c][r][i];
          z[i] = v;
          sq += v * v;
        }
        if constexpr (EXACT) {
          // k_gemm's order: the tile row's 16 squares added one after another
          sq = 0.f;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v = __shfl(z[i], lane % 16 + 16 * qq);
              sq += v * v;
            }
        } else {
          sq = xor16_sum(sq);
          sq = xor32_sum(sq);
        }
        if (ok) {
          bf16_t v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a.h[(size_t)m * a.hidden + n0 + i] = z[i];
            v[i] = f2h(z[i] * gv[i]);
          }
          if (a.opk) {
            st4h(reinterpret_cast<bf16_t*>(a.xg_out) + pk_off(m, n0, a.hidden), v);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<bf16_t*>(a.xg_out)[(size_t)m * a.hidden + n0 + i] = v[i];
          }
          if (q == 0) a.ssq_out[(size_t)m * a.ssq_ld + tg] = sq;
        }
      }
    }
  }
  stamp_end(a.stamp);
}

// Residual update after a K-split GEMM: h += sum of the S partial sums (in
// split order), then the next GEMM's input xg = h * gain_next and the
// per-16-column sums of squares of h.  Grid (M, hidden / 64), 64 threads.
template <typename T>
__global__ __launch_bounds__(64) void k_resid_reduce(GemmArgs a) {
  constexpr int SMAX = 8;
  stamp_begin(a.stamp);
  const int m = blockIdx.x, col = blockIdx.y * 64 + threadIdx.x;
  float p[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) p[s] = s < a.S ? a.part[((size_t)s * a.M + m) * a.part_ld + col] : 0.f;
  const float h0 = a.h[(size_t)m * a.hidden + col];
  const float g = a.gain_next[col];
  float v = p[0];
#pragma unroll
  for (int s = 1; s < SMAX; ++s)
    if (s < a.S) v += p[s];
  v = h0 + v;
  a.h[(size_t)m * a.hidden + col] = v;
  reinterpret_cast<T*>(a.xg_out)[(size_t)m * a.hidden + col] = Act<T>::from_f(v * g);
  float sq = v * v;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o);
  if (threadIdx.x % 16 == 0) a.ssq_out[(size_t)m * a.ssq_ld + col / 16] = sq;
  stamp_end(a.stamp);
}

// ---------------------------------------------------------------------------
// Greedy argmax over the vocabulary without [M], lowest id on ties, with the
// runner-up value (GravityOCR review, section 2 "Speculative Decoding":
// greedy top-1 verification).  Merging (top1 value, top1 id, top2 value)
// records is associative and commutative, so any reduction tree gives the
// same bits.  A NaN anywhere makes the row's record NaN.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_argmax(const float* v1, const int32_t* i1, const float* v2,
                                                    const float* gs, float sc, int n_groups, int ld, int32_t* tok,
                                                    float* top1, float* top2, float* zs, ProfStamp* stamp,
                                                    const int* err) {
  stamp_begin(stamp);
  __shared__ Top2 sh[kThreads];
  __shared__ float ssum[kThreads];
  const int m = blockIdx.x;
  constexpr int BATCH = 16;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  for (int g0 = threadIdx.x; g0 < n_groups; g0 += BATCH * kThreads) {
    Top2 rec[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int g = g0 + b * kThreads;
      rec[b] = Top2{-INFINITY, 0x7fffffff, -INFINITY};
      if (g < n_groups) rec[b] = Top2{v1[(size_t)m * ld + g], i1[(size_t)m * ld + g], v2[(size_t)m * ld + g]};
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) t = merge_top2(t, rec[b]);
  }
  // The merged record depends on the set of records only (largest value, lowest id among equal
  // maxima, second value of the multiset, NaN if any is NaN), so the merge runs in any order:
  // across each wave by shuffles, then across the waves in LDS (one barrier).
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const Top2 other{__shfl_xor(t.v1, o), __shfl_xor(t.i1, o), __shfl_xor(t.v2, o)};
    t = merge_top2(t, other);
  }
  if (threadIdx.x % kWave == 0) sh[threadIdx.x / kWave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    Top2 r = sh[0];
    for (int w = 1; w < kThreads / kWave; ++w) r = merge_top2(r, sh[w]);
    sh[0] = r;
    tok[m] = (err && *err) ? -1 : r.i1;   // a failed layer-tail barrier: no valid token
    top1[m] = r.v1;
    top2[m] = r.v2;
  }
  if (gs) {
    // the row's softmax denominator relative to its max, [M] excluded: the sum over groups of
    // gs_g * exp((v1_g - max) / T), groups in a fixed thread order and tree.  At T = 1 its
    // inverse is the greedy token's softmax probability.
    __syncthreads();   // the merged record in sh[0]
    const float mx = sh[0].v1;
    float part = 0.f;
    for (int g = threadIdx.x; g < n_groups; g += kThreads) {
      const float gv = v1[(size_t)m * ld + g];
      if (gv > -INFINITY) part += gs[(size_t)m * ld + g] * __builtin_amdgcn_exp2f((gv - mx) * sc);
    }
    ssum[threadIdx.x] = part;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (threadIdx.x < s) ssum[threadIdx.x] += ssum[threadIdx.x + s];
      __syncthreads();
    }
    if (threadIdx.x == 0) zs[m] = sh[0].i1 >= 0 ? ssum[0] : NAN;
  }
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// Block-mask attention over the paged KV cache.
// Grid: (key chunk slot, kv head, row task).  A workgroup takes up to 48 rows
// of one request, all query heads of one KV head (GQA), and the keys of
// 64-position chunks.  For each (row, head) and chunk it computes the
// chunk-local max m_c, sum l_c = sum exp(s - m_c) and o_c = sum exp(s - m_c) v
// over the keys the row may see (key <= lim[row]); invisible keys contribute
// exactly zero.  Decode forwards write one record per chunk (fold = 0) and
// k_attn_combine adds them in chunk order; prefill (fold = 1) loops over the
// chunks in the same order and writes the normalized output directly.
// S^T = K Q^T puts keys on the matrix-core row side so the probabilities land
// in the lanes that feed P^T to the V^T P^T product without shuffles; V is
// stored transposed in LDS so a V^T fragment is one or two vector reads.
// ---------------------------------------------------------------------------
// Online-softmax merge of a running (m, l, o) with a chunk record (mc, lc, oc), maxima in
// log2 units: m' = max(m, mc), l' = l 2^(m-m') + lc 2^(mc-m'), o' likewise.
__device__ __forceinline__ void fold_coef(float m, float mc, float& mn, float& al, float& be) {
  mn = fmaxf(m, mc);
  al = __builtin_amdgcn_exp2f(m - mn);     // m = -inf (empty running state) gives 0
  be = __builtin_amdgcn_exp2f(mc - mn);
}
// Two fp32 values rounded to fp16 (nearest even) and packed, low half first.
__device__ __forceinline__ uint32_t pack_h2(float x, float y) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  const f32x2v f = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2v));
}
__device__ __forceinline__ float fold_val(float v, float al, float vc, float be) {
  return __fadd_rn(__fmul_rn(v, al), __fmul_rn(vc, be));
}

// fp16 K/V: at most 128 VGPRs, so four workgroups share a CU (long contexts launch several per CU).
// Folded rows (FOLD) run fold_streams<T>() chunk streams of four waves each (stream k takes
// chunks k, k + streams, ...) of the same rows and heads, and merge the running states into
// stream 0's at the end, in stream order: a fraction of the dependent chain per workgroup and
// several waves per SIMD (two streams: 28.6 -> 20.5 us per 1088-row prefill layer).  fp32 K/V
// keeps two streams (four would spill).
template <typename T>
constexpr int fold_streams() { return sizeof(T) == 2 ? 4 : 2; }
template <typename T, int HD, bool FOLD>
__global__ __launch_bounds__((FOLD ? fold_streams<T>() : 1) * kAttnThreads,
                             (FOLD ? fold_streams<T>() : (sizeof(T) == 2 ? 4 : 1))) void k_attn(AttnArgs a) {
#pragma clang fp contract(off)
  constexpr int NTH = kAttnThreads;        // threads of one chunk stream
  constexpr int NST = FOLD ? fold_streams<T>() : 1;   // chunk streams
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int DT = HD / 16;
  constexpr int QKS = HD / KS;             // steps of S^T over the head dimension
  constexpr int KT = kKeyChunk / 16;       // key tiles per chunk
  constexpr int PVS = kKeyChunk / KS;      // steps of P V over keys
  constexpr int KSTR = HD * (int)sizeof(T) + 16;              // K rows [key][d]
  constexpr int VSTR = kKeyChunk * (int)sizeof(T) + 16;      // V^T rows [d][key] (16-byte aligned)
  constexpr int TILES = kTaskRows / 16;    // 16-row tiles per task
  constexpr int REC = HD + 4;
  constexpr int FPK = HD / PER;            // 16-byte fragments per key row
  constexpr int NKF = 2 * kKeyChunk * FPK; // K and V fragments of one chunk
  // Fragment f < kKeyChunk * FPK is K: key f / FPK, dims (f % FPK) * PER.. (token-major blocks).
  // The rest are V, read from dim-major page blocks in memory order: page pc of the chunk,
  // dim d, tokens g * PER.. (PER consecutive keys of one dim: a V^T row piece).
  constexpr int GPP = kPage / PER;         // V fragments per (page, dim)
  auto frag_key = [](int f) {
    const int rem = f % (kKeyChunk * FPK);
    return f < kKeyChunk * FPK ? rem / FPK : rem / (HD * GPP) * kPage + rem % GPP * PER;
  };
  constexpr int KVF = NKF / NTH;
  static_assert(NKF % NTH == 0, "every thread loads the same number of K/V fragments");
  __shared__ __align__(16) unsigned char ks[NST * kKeyChunk * KSTR];
  __shared__ __align__(16) unsigned char vts[NST * HD * VSTR];
  __shared__ int s_lim[16];
  // the other streams' running states go to stream 0 through the K buffers after the loop
  static_assert(!FOLD || NST * kKeyChunk * KSTR >= (kAttnThreads / kWave) * kWave * (4 * DT + 2) * 4, "state exchange");

  stamp_begin(a.stamp);
  // folded rows: the tiles of the longest key ranges (the last rows) are dispatched first, so the
  // workgroups left for a second wave of the grid are short ones
  const int zi = FOLD ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.z;
  const AttnTask task = a.tasks.t[zi / TILES];
  const int mt = zi % TILES;               // this workgroup's 16-row tile of the task
  if (mt * 16 >= task.nrows) return;
  const int g = blockIdx.y;
  const int sm = (int)threadIdx.x / NTH;   // chunk stream (0 unless FOLD)
  const int tl = (int)threadIdx.x % NTH;   // thread within the stream
  unsigned char* const ksm = ks + sm * kKeyChunk * KSTR;
  unsigned char* const vtsm = vts + sm * HD * VSTR;
  const int wave = tl / kWave, lane = tl % kWave;
  const int n_rep = a.n_heads / a.n_kv;
  const bool active = wave < n_rep;        // wave = query head within the KV group
  const int row_local = mt * 16 + lane % 16;
  const int head = g * n_rep + wave;
  const int32_t* pt = a.fwd_pt + (size_t)task.req * a.pt_ld;
  // scores are kept in log2 units: s * scale * log2(e), so the softmax uses exp2
  const float qscale = a.scale * kLog2e;

  // ---- first memory round trip: page ids, limits, query fragments (loads complete in issue
  //      order, so the K/V addresses wait for the page ids only) ----
  const int cbeg = FOLD ? 0 : blockIdx.x;
  int pg[KVF];
  {
    const int c1 = min(cbeg + sm, a.max_chunks - 1);   // this stream's first chunk (a junk one past the end)
#pragma unroll
    for (int q = 0; q < KVF; ++q) pg[q] = pt[(c1 * kKeyChunk + frag_key(tl + q * NTH)) / kPage];
  }
  // Branch-free as well (clamped to the task's last row and the last head): rows past the task
  // and idle waves read real data that never reaches a written result (rows stay independent in
  // both products; idle waves skip them).
  const int lim_row = mt * 16 + (int)threadIdx.x % 16;
  const int lim_ld = a.row_lim[task.row0 + min(lim_row, task.nrows - 1)];
  uint4 qf[QKS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (size_t)(task.row0 + min(row_local, task.nrows - 1)) * a.q_ld +
                  min(head, a.n_heads - 1) * HD + PER * (lane / 16);
#pragma unroll
    for (int st = 0; st < QKS; ++st) qf[st] = *reinterpret_cast<const uint4*>(qp + st * KS);
  }
  // largest visibility limit of the task's rows
  const int maxlim = task.lim_mode == 0 ? task.max_lim : a.req->p[task.req] + a.req->B + (task.lim_mode == 2 ? 1 : 0);
  const int cend = FOLD ? maxlim / kKeyChunk + 1 : cbeg + 1;
  if (cbeg * kKeyChunk > maxlim) return;     // no visible key in this chunk slot

  float run_m = -INFINITY, run_l = 0.f;
  f32x4_t run_o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) run_o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // ---- second round trip: K and V of keys [c*64, c*64+64) ----
  // Unconditional loads: a conditional load makes the compiler wait for it inside its branch,
  // which serialised the KVF round trips.  Every address is in the pool: the page list holds
  // page 0 past the request's pages.  Keys past the task's limit are zeroed below (their
  // scores are masked; a zero V keeps 0 * P finite).
  auto load_kv = [&](const int (&pgs)[KVF], uint4 (&dst)[KVF]) {
#pragma unroll
    for (int q = 0; q < KVF; ++q) {
      const int f = tl + q * NTH;
      const int kv = f / (kKeyChunk * FPK);
      const int rem = f % (kKeyChunk * FPK);
      const int key = frag_key(f) % kPage, dim = kv == 0 ? (rem % FPK) * PER : rem % (HD * GPP) / GPP;
      dst[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.kv_pool) +
                                               kv_off(a.layer, a.n_pages, pgs[q], kv, a.n_kv, g, key, dim, HD));
    }
  };
  auto load_pg = [&](int c, int (&dst)[KVF]) {
#pragma unroll
    for (int q = 0; q < KVF; ++q) dst[q] = pt[(c * kKeyChunk + frag_key(tl + q * NTH)) / kPage];
  };
  // Folded rows walk their chunks with the next chunk's K and V and the page ids of the one after
  // in flight while the current chunk is multiplied (the last chunks re-read the last one, never
  // used), so a chunk costs its products rather than two dependent memory round trips.
  uint4 kvv[KVF];
  load_kv(pg, kvv);
  if constexpr (FOLD) load_pg(min(cbeg + sm + NST, cend - 1), pg);

  for (int c0 = cbeg; c0 < cend; c0 += NST) {
    const int c = c0 + sm;                 // this stream's chunk
    const bool cvalid = c < cend;          // (later streams may have none in the last pass)
    // (the row limits are stored once the K/V loads are in flight)
    if (threadIdx.x < 16) s_lim[threadIdx.x] = lim_row < task.nrows ? lim_ld : -1;
#pragma unroll
    for (int q = 0; q < KVF; ++q) {
      const int f = tl + q * NTH;
      const int kv = f / (kKeyChunk * FPK);
      const int rem = f % (kKeyChunk * FPK);
      const int kk = frag_key(f);
      if (kv == 0) {
        if (c * kKeyChunk + kk > maxlim) kvv[q] = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(ksm + kk * KSTR + (rem % FPK) * PER * (int)sizeof(T)) = kvv[q];
      } else {
        // zero the values of keys past the limit (PER keys per fragment)
        const int nv = maxlim - (c * kKeyChunk + kk) + 1;
        uint32_t* wv = reinterpret_cast<uint32_t*>(&kvv[q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (sizeof(T) == 2) {
            if (2 * i >= nv) wv[i] = 0;
            else if (2 * i + 1 >= nv) wv[i] &= 0xffffu;
          } else {
            if (i >= nv) wv[i] = 0;
          }
        }
        const int d = rem % (HD * GPP) / GPP;
        *reinterpret_cast<uint4*>(vtsm + d * VSTR + kk * (int)sizeof(T)) = kvv[q];
      }
    }
    __syncthreads();
    if constexpr (FOLD) {
      load_kv(pg, kvv);                        // chunk c + NST (its page ids landed a pass ago)
      load_pg(min(c + 2 * NST, cend - 1), pg);
    }

    if (active && cvalid) {
      // S^T tiles: element i of tile kt = score of key kt*16 + 4*(lane/16) + i for row_local
      f32x4_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QKS; ++st) {
          const uint4 kf = *reinterpret_cast<const uint4*>(
              ksm + (kt * 16 + lane % 16) * KSTR + (st * KS + PER * (lane / 16)) * (int)sizeof(T));
          mma_aa(s[kt], kf, qf[st], T());
        }
      }
      const int lim = s_lim[lane % 16];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = c * kKeyChunk + kt * 16 + 4 * (lane / 16) + i;
          const float z = key <= lim ? s[kt][i] * qscale : -INFINITY;
          s[kt][i] = z;
          mx = fmaxf(mx, z);
        }
      mx = xor16_max(mx);
      mx = xor32_max(mx);
      // a row with no visible key in this chunk has mx = -inf and contributes nothing
      const float mref = mx == -INFINITY ? 0.f : mx;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[kt][i] - mref);   // exp2(-inf) = 0
          s[kt][i] = p;
          lsum += p;
        }
      lsum = xor16_sum(lsum);
      lsum = xor32_sum(lsum);
      // o^T = V^T P^T ; lane supplies keys pi(lane, j) for P^T and V^T alike
      f32x4_t o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < PVS; ++st) {
        uint4 pf;
        if constexpr (sizeof(T) == 2) {
          // keys 32st + 4(l/16) + {0..3} from tile 2st, then the same +16 from tile 2st+1
          const f32x4_t p0 = s[2 * st], p1 = s[2 * st + 1];
          pf.x = pack_h2(p0[0], p0[1]);
          pf.y = pack_h2(p0[2], p0[3]);
          pf.z = pack_h2(p1[0], p1[1]);
          pf.w = pack_h2(p1[2], p1[3]);
        } else {
          const f32x4_t p0 = s[st];
          pf = make_uint4(__float_as_uint(p0[0]), __float_as_uint(p0[1]), __float_as_uint(p0[2]),
                          __float_as_uint(p0[3]));
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const unsigned char* vrow = vtsm + (dt * 16 + lane % 16) * VSTR;
          uint4 vf;
          if constexpr (sizeof(T) == 2) {
            const uint2 va = *reinterpret_cast<const uint2*>(vrow + (32 * st + 4 * (lane / 16)) * 2);
            const uint2 vb = *reinterpret_cast<const uint2*>(vrow + (32 * st + 16 + 4 * (lane / 16)) * 2);
            vf = make_uint4(va.x, va.y, vb.x, vb.y);
          } else {
            vf = *reinterpret_cast<const uint4*>(vrow + (16 * st + 4 * (lane / 16)) * 4);
          }
          mma_aa(o[dt], vf, pf, T());
        }
      }
      // o[dt][i] = o_c[d = dt*16 + 4*(lane/16) + i] of row_local; the record's max is mref
      if constexpr (FOLD) {
        if (mx != -INFINITY) {
          float mn, al, be;
          fold_coef(run_m, mref, mn, al, be);
          run_l = fold_val(run_l, al, lsum, be);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) run_o[dt][i] = fold_val(run_o[dt][i], al, o[dt][i], be);
          run_m = mn;
        }
      } else if (row_local < task.nrows) {
        float* rec = a.part + (((size_t)(task.row0 + row_local) * a.n_heads + head) * a.max_chunks + c) * REC;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4_t*>(rec + dt * 16 + 4 * (lane / 16)) = o[dt];
        if (lane < 16) *reinterpret_cast<float2*>(rec + HD) = make_float2(mx, lsum);
      }
    }
    __syncthreads();
  }

  if constexpr (FOLD) {
    // streams 1, 2, ... hand their (m, l, o) to stream 0 in turn, merged by the same online step
    constexpr int XS = 4 * DT + 2;
    float* xs = reinterpret_cast<float*>(ks) + (size_t)(wave * kWave + lane) * XS;
    for (int k = 1; k < NST; ++k) {
      if (sm == k) {
        xs[0] = run_m;
        xs[1] = run_l;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xs[2 + 4 * dt + i] = run_o[dt][i];
      }
      __syncthreads();
      const float m1 = xs[0];
      if (sm == 0 && m1 != -INFINITY) {
        float mn, al, be;
        fold_coef(run_m, m1, mn, al, be);
        run_l = fold_val(run_l, al, xs[1], be);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) run_o[dt][i] = fold_val(run_o[dt][i], al, xs[2 + 4 * dt + i], be);
        run_m = mn;
      }
      __syncthreads();   // before the next stream overwrites the exchange area
    }
  }

  if (FOLD && sm == 0 && active && row_local < task.nrows) {
    const int row = task.row0 + row_local;
    T* dst = reinterpret_cast<T*>(a.out) + (size_t)row * a.out_ld + head * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      T v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = Act<T>::from_f(run_o[dt][i] / run_l);
      if (sizeof(T) == 2 && a.opk) {   // four consecutive values of one 8-value group: one 8-byte store
        st4h(reinterpret_cast<T*>(a.out) + pk_off(row, head * HD + dt * 16 + 4 * (lane / 16), a.out_ld), v);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[dt * 16 + 4 * (lane / 16) + i] = v[i];
      }
    }
  }
  stamp_end(a.stamp);
}

// Combine the per-chunk records of each (row, head).  One wave per (row,
// head); lane d holds output dimension d.  The row's limit and up to 32
// records are loaded in one round trip; records of chunks past the limit
// were never written and are replaced by empty ones.  Within a batch of 32
// chunks: m* = max m_c, then l = sum l_c 2^(m_c - m*) and
// o = sum o_c 2^(m_c - m*) in chunk order (maxima in log2 units); batches fold online.
template <typename T, int HD>
__global__ __launch_bounds__(kWave) void k_attn_combine(const float* part, int max_chunks, int n_slots,
                                                          int n_heads, const int32_t* row_lim, int M, void* out,
                                                          int out_ld, ProfStamp* stamp) {
  stamp_begin(stamp);
  constexpr int REC = HD + 4;
  constexpr int BATCH = 32;
  const int lane = threadIdx.x;
  const int idx = blockIdx.x;
  if (idx >= M * n_heads) return;
  const int row = idx / n_heads, head = idx % n_heads;
  const int lim = row_lim[row];
  const float* rec = part + ((size_t)row * n_heads + head) * max_chunks * REC;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int c0 = 0; c0 < n_slots; c0 += BATCH) {
    float mc[BATCH], lc[BATCH], oc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = min(c0 + b, n_slots - 1);
      const float2 ml = *reinterpret_cast<const float2*>(rec + c * REC + HD);
      mc[b] = ml.x; lc[b] = ml.y;
      oc[b] = rec[c * REC + min(lane, HD - 1)];
    }
    // chunks that hold a visible key of this row; the empty asm keeps this (loop-invariant) use of
    // the limit inside the loop, so the record loads above are issued before the limit is awaited
    int limv = lim;
    asm volatile("" : "+v"(limv));
    const int nvis = limv / kKeyChunk + 1;
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (c0 + b >= nvis || c0 + b >= n_slots) { mc[b] = -INFINITY; lc[b] = 0.f; oc[b] = 0.f; }
      mx = fmaxf(mx, mc[b]);
    }
    if (mx == -INFINITY) continue;
    float lb = 0.f, ob = 0.f;
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const float w = __builtin_amdgcn_exp2f(mc[b] - mx);
      lb = __fadd_rn(lb, __fmul_rn(lc[b], w));
      ob = __fadd_rn(ob, __fmul_rn(oc[b], w));
    }
    if (m == -INFINITY) {
      m = mx; l = lb; o = ob;
    } else {
      float mn, al, be;
      fold_coef(m, mx, mn, al, be);
      l = fold_val(l, al, lb, be);
      o = fold_val(o, al, ob, be);
      m = mn;
    }
  }
  if (lane < HD) reinterpret_cast<T*>(out)[(size_t)row * out_ld + head * HD + lane] = Act<T>::from_f(o / l);
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// Accept + commit (GravityOCR review, section 3.2 and Appendix B.2): one wave
// per request.  Lane j compares d_{j+1} (verify input row j+1) with a_{j+1}
// (verify argmax of row j); A = index of the first mismatch (B if none).  The
// round commits a0, a_1..a_{A+1} (= a0, d_1..d_A, a_{A+1}), cut after the
// first EOS and at the output budget; a_{A+1} becomes the next boundary.
// Output per request: [A, n_committed, next_x0, eos_seen, committed...].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_accept(const int32_t* row_tok, const int32_t* am, const ReqArgs* rap,
                                               int eos_id, int32_t* out, int out_stride, const int* err,
                                               ProfStamp* stamp) {
  stamp_begin(stamp);
  const ReqArgs& ra = *rap;
  const int r = blockIdx.x, j = threadIdx.x;
  const int B = ra.B, row0 = ra.row0[r];
  // Every load is unconditional (indices clamped into the request's B + 1 rows), so the few
  // round trips overlap instead of each being awaited inside its own branch.
  const int dj = row_tok[min(row0 + 1 + j, row0 + B)], aj = am[min(row0 + j, row0 + B)];
  const unsigned long long bal = __ballot(j < B && dj != aj);
  const int A = bal ? __builtin_ctzll(bal) : B;
  int32_t* o = out + (size_t)r * out_stride;
  // candidate commit list: k = 0 -> a0, k >= 1 -> a_k = am[row0 + k - 1]; lane j holds
  // candidates j and j + 64, the first EOS among them cuts the list
  const int ncand = A + 2;
  auto cand = [&](int k) { return k == 0 ? row_tok[row0] : am[row0 + k - 1]; };
  const int k1 = j, k2 = j + 64;
  const int t1 = cand(min(k1, ncand - 1)), t2 = cand(min(k2, ncand - 1));
  const unsigned long long e1 = __ballot(k1 < ncand && t1 == eos_id);
  const unsigned long long e2 = __ballot(k2 < ncand && t2 == eos_id);
  const int eos_at = e1 ? __builtin_ctzll(e1) : (e2 ? 64 + __builtin_ctzll(e2) : ncand);
  int n = min(ncand, eos_at + 1);
  n = min(n, ra.max_commit[r]);
  if (k1 < n) o[4 + k1] = t1;
  if (k2 < n) o[4 + k2] = t2;
  if (j == 0) {
    o[0] = (err && *err) ? -1 : A;   // a failed layer-tail barrier: the host rejects the round
    o[1] = n;
    o[2] = am[row0 + A];
    o[3] = (eos_at < ncand && eos_at < n) ? 1 : 0;
  }
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// Debug poisoning of KV slots that no correct read may reach (a test of the
// in-place overwrite and of rollback): NaN into every layer's K and V at the
// positions [lo, p + B + 2) of each request, lo = p + 1 between the draft and
// the verify forward (the verify rewrites them before any read), or
// lo = p + A + 2 after accept (rolled back; the next window rewrites them).
// lo_abs >= 0 gives the range [lo_abs, hi_abs) explicitly (a test hook).
// Grid (requests x layers), 256 threads; vector stores only.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_poison_kv(const ReqArgs* rap, const int32_t* acc, int acc_stride,
                                                   int lo_abs, int hi_abs, void* kv_pool, int n_layers, int n_pages,
                                                   int n_kv, int hd) {
  const ReqArgs& ra = *rap;
  const int r = blockIdx.x / n_layers, layer = blockIdx.x % n_layers;
  const int p = ra.p[r];
  const int lo = lo_abs >= 0 ? lo_abs : acc ? p + acc[(size_t)r * acc_stride] + 2 : p + 1;
  const int hi = lo_abs >= 0 ? hi_abs : p + ra.B + 2;
  const int per = 2 * n_kv * hd;                    // K and V values of one position
  T* pool = reinterpret_cast<T*>(kv_pool);
  for (int e = threadIdx.x; e < (hi - lo) * per; e += blockDim.x) {
    const int s = lo + e / per, rem = e % per;
    const int kv = rem / (n_kv * hd), h = (rem / hd) % n_kv, d = rem % hd;
    const int pg = ra.pt[r][s / kPage];
    pool[kv_off(layer, n_pages, pg, kv, n_kv, h, s % kPage, d, hd)] = Act<T>::from_f(NAN);
  }
}

// ---------------------------------------------------------------------------
// Direct block-diffusion step (GravityOCR review, Appendix B.1; Trillion Labs
// blog, the "confidence threshold" entry): one wave per request.  Lane j owns
// block position j + 1, whose prediction is window row j.  Every undecided
// position whose confidence reaches tau is committed; when none does, the
// single most confident undecided one is (lowest position on ties).  Under a
// draft schedule (dsteps > 0; blog, the draft-schedule passage) the last
// allowed step commits every open position; slot B always receives row B's
// prediction (the schedule's d_B).
// Record per request (rec_stride ints): [committed this step, still undecided,
// invalid, steps so far, step_of[B], tokens[B], confidence bits[B], greedy
// token of every row[B]].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_dd_init(const ReqArgs* rap, int mask_id, int32_t* rec, int rec_stride) {
  const ReqArgs& ra = *rap;
  const int r = blockIdx.x, j = threadIdx.x, B = ra.B;
  int32_t* o = rec + (size_t)r * rec_stride;
  if (j < B) {
    ra.win[r][j] = mask_id;
    o[4 + j] = -1;
    o[4 + B + j] = mask_id;
  }
  if (j < 4) o[j] = 0;
}

__global__ __launch_bounds__(64) void k_dd_select(const int32_t* am, const float* zs, const ReqArgs* rap,
                                                  int mask_id, int vocab, int32_t* rec, int rec_stride) {
  const ReqArgs& ra = *rap;
  const int r = blockIdx.x, j = threadIdx.x;
  const int B = ra.B, row0 = ra.row0[r];
  int32_t* win = ra.win[r];
  int32_t* o = rec + (size_t)r * rec_stride;
  const int step = o[3];
  const bool lane = j < B;
  const int cur = lane ? win[j] : mask_id;
  const bool und = lane && cur == mask_id;
  const int tk = lane ? am[row0 + j] : 0;
  const float c = lane ? 1.0f / zs[row0 + j] : 0.f;   // softmax probability of the greedy token
  const bool bad = und && (tk < 0 || tk >= vocab || tk == mask_id || !(c >= 0.f));
  const bool final_step = ra.dsteps > 0 && step + 1 >= ra.dsteps;
  const bool hit = und && (final_step || c >= ra.tau);
  bool take = hit;
  if (__ballot(hit) == 0) {
    float bc = und ? c : -INFINITY;
    int bj = und ? j : kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float oc = __shfl_xor(bc, off);
      const int oj = __shfl_xor(bj, off);
      if (oc > bc || (oc == bc && oj < bj)) { bc = oc; bj = oj; }
    }
    take = und && j == bj;
  }
  const unsigned long long tb = __ballot(take);
  const unsigned long long ub = __ballot(und && !take);
  const int tB = am[row0 + B];
  const bool badB = ra.dsteps > 0 && (tB < 0 || tB >= vocab || tB == mask_id);
  const unsigned long long bb = __ballot(bad || (j == 0 && badB));
  if (take && !bb) win[j] = tk;
  if (j == 0 && !bb) win[B] = tB;
  if (lane) {
    if (take) o[4 + j] = step;
    o[4 + B + j] = take ? tk : cur;
    o[4 + 2 * B + j] = __float_as_int(c);
    o[4 + 3 * B + j] = tk;
  }
  if (j == 0) {
    o[0] = __popcll(tb);
    o[1] = __popcll(ub);
    o[2] = bb ? 1 : 0;
    o[3] = step + 1;
  }
}

// ---------------------------------------------------------------------------
// Stochastic rounds (GravityOCR review, section 2 "Speculative Decoding";
// Trillion Labs blog, the speculative rejection rule preserving the sampling
// distribution).  Draws are inverse-CDF over token ids in increasing order:
// the smallest id whose cumulative mass exceeds u times the total.
// ---------------------------------------------------------------------------

// Inclusive scan of one value per thread over the workgroup, in a fixed
// (Hillis-Steele) order; sh[t] holds thread t's inclusive sum on return.
__device__ __forceinline__ float block_incl_scan(float v, float* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const float o = t >= off ? sh[t - off] : 0.f;
    __syncthreads();
    sh[t] += o;
    __syncthreads();
  }
  return sh[t];
}

// One row's draw from softmax(z / T) without [M].  The row's mass is split by
// LM-head column group (group g holds gs_g * exp((v1_g - max) / T)): thread i
// adds a contiguous run of groups in id order, a workgroup scan of the runs
// finds the group where u * S falls (S: the row's total), and one wave scans
// that group's columns in id order.  Where rounding leaves u * S past the last
// cumulative value, the last group / column of positive mass is taken.
// Grid (rows per request, requests); row j of request r draws with u[r][j].
__global__ __launch_bounds__(kThreads) void k_sample_rows(SampleArgs a) {
  __shared__ float sh[kThreads];
  __shared__ int s_thr, s_last, s_grp;
  __shared__ float s_base;
  const ReqArgs& ra = *a.req;
  const int r = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int m = ra.row0[r] + j;
  const float mx = a.rmax[m];
  const float target = ra.u[r][j] * a.rz[m];
  const int G = (a.n_groups + kThreads - 1) / kThreads, g0 = t * G;
  const float* v1 = a.v1 + (size_t)m * a.ld;
  const float* gs = a.gs + (size_t)m * a.ld;
  auto mass = [&](int g) -> float {
    const float gv = v1[g];
    return gv > -INFINITY ? gs[g] * __builtin_amdgcn_exp2f((gv - mx) * a.sc) : 0.f;
  };
  float loc = 0.f;
  for (int k = 0; k < G; ++k)
    if (g0 + k < a.n_groups) loc += mass(g0 + k);
  if (t == 0) { s_thr = 0x7fffffff; s_last = -1; s_grp = -1; s_base = 0.f; }
  const float incl = block_incl_scan(loc, sh);
  const float excl = t ? sh[t - 1] : 0.f;
  if (loc > 0.f && excl <= target && target < incl) atomicMin(&s_thr, t);
  if (loc > 0.f) atomicMax(&s_last, t);
  __syncthreads();
  if (t == (s_thr != 0x7fffffff ? s_thr : s_last)) {
    float cum = excl, base_last = excl;
    int grp = -1, last = -1;
    for (int k = 0; k < G && g0 + k < a.n_groups; ++k) {
      const float c = mass(g0 + k);
      if (c > 0.f) {
        last = g0 + k;
        base_last = cum;
        if (cum + c > target) { grp = g0 + k; break; }
      }
      cum += c;
    }
    if (grp < 0) { grp = last; cum = base_last; }
    s_grp = grp;
    s_base = cum;
  }
  __syncthreads();
  if (t < kWave) {
    const int grp = s_grp;     // -1 only for a row without positive mass (NaN logits)
    const int col = grp * a.gcols + t;
    float e = 0.f;
    if (grp >= 0 && t < a.gcols && col < a.vocab && col != a.mask_id)
      e = __builtin_amdgcn_exp2f((a.logits[(size_t)m * a.vocab + col] - mx) * a.sc);
    float cs = e;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(cs, off);
      if (t >= off) cs += o;
    }
    const unsigned long long hit = __ballot(e > 0.f && s_base + cs > target);
    const unsigned long long pos = __ballot(e > 0.f);
    const int pick = hit ? __builtin_ctzll(hit) : (pos ? 63 - __builtin_clzll(pos) : -1);
    if (t == 0) a.tok[m] = (grp >= 0 && pick >= 0) ? grp * a.gcols + pick : -1;
  }
}

// Acceptance test and the next token of a stochastic round, one workgroup per
// request.  Wave 0: lane j tests d_{j+1} (verify input row j+1): accepted iff
// u_acc * q(d) < p(d), p from verify row j, q from draft row j+1; A = number
// accepted before the first rejection.  Then the whole workgroup draws the
// next token t: from max(0, p - q) at verify row A / draft row A+1 when
// A < B (from p alone if that residual has no mass), from verify row B when
// A = B; thread i adds a contiguous run of token ids, a workgroup scan finds
// where u_t times the total falls.  Commit record as k_accept.
__global__ __launch_bounds__(kThreads) void k_accept_sample(AcceptSampleArgs a) {
  __shared__ float sh[kThreads];
  __shared__ int s_A, s_thr, s_last, s_pick;
  const ReqArgs& ra = *a.req;
  const int r = blockIdx.x, t = threadIdx.x;
  const int B = ra.B, row0 = ra.row0[r];
  const float* u = ra.u[r];
  const size_t V = (size_t)a.vocab;
  if (t < kWave) {
    bool rej = false;
    if (t < B) {
      const int d = a.row_tok[row0 + 1 + t];
      const int pr = row0 + t, qr = row0 + t + 1;
      const float p = __builtin_amdgcn_exp2f((a.lg_v[pr * V + d] - a.vmax[pr]) * a.sc) / a.vz[pr];
      const float q = __builtin_amdgcn_exp2f((a.lg_d[qr * V + d] - a.dmax[qr]) * a.sc) / a.dz[qr];
      rej = !(u[B + 1 + t] * q < p);
    }
    const unsigned long long b = __ballot(rej);
    if (t == 0) { s_A = b ? __builtin_ctzll(b) : B; s_pick = -1; }
  }
  __syncthreads();
  const int A = s_A;
  const int pr = row0 + A, qr = row0 + A + 1;
  const float pm = a.vmax[pr], pinv = 1.0f / a.vz[pr];
  const float qm = A < B ? a.dmax[qr] : 0.f, qinv = A < B ? 1.0f / a.dz[qr] : 0.f;
  const int chunk = (a.vocab + kThreads - 1) / kThreads;
  const int v0 = min(t * chunk, a.vocab), v1 = min(a.vocab, v0 + chunk);
  auto w = [&](int v, bool useq) -> float {
    if (v == a.mask_id) return 0.f;
    const float p = __builtin_amdgcn_exp2f((a.lg_v[pr * V + v] - pm) * a.sc) * pinv;
    if (!useq) return p;
    const float q = __builtin_amdgcn_exp2f((a.lg_d[qr * V + v] - qm) * a.sc) * qinv;
    return fmaxf(p - q, 0.f);
  };
  for (int attempt = 0; attempt < 2; ++attempt) {
    const bool useq = A < B && attempt == 0;
    float loc = 0.f;
    for (int v = v0; v < v1; ++v) loc += w(v, useq);
    if (t == 0) { s_thr = 0x7fffffff; s_last = -1; }
    const float incl = block_incl_scan(loc, sh);
    const float excl = t ? sh[t - 1] : 0.f;
    const float tot = sh[kThreads - 1];
    if (!(tot > 0.f)) {      // same value in every thread: a uniform branch
      __syncthreads();
      continue;
    }
    const float target = u[2 * B + 1] * tot;
    if (loc > 0.f && excl <= target && target < incl) atomicMin(&s_thr, t);
    if (loc > 0.f) atomicMax(&s_last, t);
    __syncthreads();
    if (t == (s_thr != 0x7fffffff ? s_thr : s_last)) {
      float cum = excl;
      int pick = -1, last = -1;
      for (int v = v0; v < v1; ++v) {
        const float x = w(v, useq);
        if (x > 0.f) {
          last = v;
          if (cum + x > target) { pick = v; break; }
        }
        cum += x;
      }
      s_pick = pick >= 0 ? pick : last;
    }
    break;
  }
  __syncthreads();
  if (t == 0) {
    const int tk = s_pick;
    int32_t* o = a.out + (size_t)r * a.out_stride;
    const int ncand = A + 2;
    int eos_at = ncand;
    for (int k = 0; k < ncand; ++k) {
      const int x = k <= A ? a.row_tok[row0 + k] : tk;
      if (x == a.eos_id) { eos_at = k; break; }
    }
    int n = min(ncand, eos_at + 1);
    n = min(n, ra.max_commit[r]);
    for (int k = 0; k < n; ++k) o[4 + k] = k <= A ? a.row_tok[row0 + k] : tk;
    o[0] = (a.err && *a.err) ? -1 : A;   // a failed layer-tail barrier: the host rejects the round
    o[1] = n;
    o[2] = tk;
    o[3] = (eos_at < ncand && eos_at < n) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (C++ linkage, used by the engine).
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_pack(uint4* dst, int n_tiles, int K, int mode, const void* s0, const void* s1,
                       const void* s2, int n0, int n1, int hd, int* range_err, hipStream_t st) {
  hipLaunchKernelGGL(k_pack<T>, dim3(1024), dim3(256), 0, st, dst, n_tiles, K, mode,
                     (const T*)s0, (const T*)s1, (const T*)s2, n0, n1, hd, range_err);
  return hipGetLastError();
}
template hipError_t launch_pack<bf16_t>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                        int, int, int*, hipStream_t);
template hipError_t launch_pack<float>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                       int, int, int*, hipStream_t);

template <typename T>
hipError_t launch_prep(const PrepArgs& a, hipStream_t st) {
  SSB_LAUNCH(k_prep_embed<T>, dim3(a.M, a.hidden / 64), dim3(64), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_prep<bf16_t>(const PrepArgs&, hipStream_t);
template hipError_t launch_prep<float>(const PrepArgs&, hipStream_t);

template <typename T, int EPI, int MT, int KPW>
static hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t st) {
  const int KR = a.KSL * KPW * Ty<T>::kStepK;
  const GemmLds L = gemm_lds(MT, KR * (int)sizeof(T), a.NT, a.KSL, a.n_ssq, EPI);
  const int m_blocks = (a.M + 16 * MT - 1) / (16 * MT);
  int gx = a.n_tiles / a.NT;
  if constexpr (MT == 3 || MT == 1) {
    if (m_blocks >= 5) {
      // many row blocks: one tile group per workgroup, which walks gz-strided row blocks with
      // its weights held in registers.  One such workgroup fits a CU (LDS and registers), so
      // the grid stays within one workgroup per CU; 48-row blocks keep at least two per
      // workgroup.  (With up to 3 row blocks the parallel grid measured faster; from 5 the loop
      // wins, by 6% at 198 rows, 13-15% at 264-528 and 18% at 1040.  The 16-row blocks of the
      // 4096-long down projection spread as widely as the CUs allow.)
      const int want = kGemmPersistentWgs / (gx * a.S);
      const int gz = max(1, min(want, MT == 1 ? m_blocks : m_blocks / 2));
      const dim3 grid(gx, a.S, gz), block(kGemmThreads);
      SSB_LAUNCH((k_gemm<T, MT, EPI, KPW, true>), grid, block, L.total, st, a);
      return hipGetLastError();
    }
  }
  if (EPI == EPI_LOGITS) {           // persistent: about one workgroup per CU, equal group counts
    const int per = (gx + kGemmPersistentWgs - 1) / kGemmPersistentWgs;
    gx = (gx + per - 1) / per;
  }
  const dim3 grid(gx, a.S, m_blocks), block(kGemmThreads);
  SSB_LAUNCH((k_gemm<T, MT, EPI, KPW, false>), grid, block, L.total, st, a);
  return hipGetLastError();
}

template <typename T, int EPI, int MT>
static hipError_t launch_gemm_mt(const GemmArgs& a, hipStream_t st) {
  const int kpw = a.K / a.S / Ty<T>::kStepK / a.KSL;      // K steps per wave
  if constexpr (sizeof(T) == 2) {
    switch (kpw) {
      case 4: return launch_gemm_cfg<T, EPI, MT, 4>(a, st);
      case 8: return launch_gemm_cfg<T, EPI, MT, 8>(a, st);
      case 16: return launch_gemm_cfg<T, EPI, MT, 16>(a, st);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kpw) {
      case 1: return launch_gemm_cfg<T, EPI, MT, 1>(a, st);
      case 2: return launch_gemm_cfg<T, EPI, MT, 2>(a, st);
      case 4: return launch_gemm_cfg<T, EPI, MT, 4>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
}

// Largest row-tile count MT <= 3 whose LDS fits (0: none fits).
int gemm_max_mt(int elem, int K, int S, int NT, int KSL, int n_ssq, int epi) {
  for (int mt = 3; mt >= 1; --mt)
    if (gemm_lds(mt, K / S * elem, NT, KSL, n_ssq, epi).total <= kGemmMaxLds) return mt;
  return 0;
}

template <typename T, int EPI>
static hipError_t launch_gemm_epi(const GemmArgs& a, hipStream_t st) {
  const int fit = gemm_max_mt((int)sizeof(T), a.K, a.S, a.NT, a.KSL, a.n_ssq, EPI);
  if (fit == 0 || a.NT * a.KSL > kGemmThreads / kWave || a.n_tiles % a.NT != 0 || a.n_ssq > kMaxNormParts ||
      a.n_ssq % 8 != 0)
    return hipErrorInvalidValue;
  // Row tile height never changes a row's arithmetic (each row's K slices are summed in the same
  // order), only the launch shape.  The smallest tile whose grid still fits one workgroup per CU
  // runs fastest: more, shorter blocks spread the slab staging over more CUs, while a grid past
  // one workgroup per CU (the slab leaves room for one) runs in two rounds.  At 33 rows: QKV in
  // 32-row blocks (192 workgroups; 7.8 -> 7.3 us against 48-row blocks, 7.9 in 16-row blocks),
  // O in 16-row blocks (192; 7.3 -> 6.4 us), gate|up in 48-row blocks (256; 13.3 us in 32-row).
  // (Never taller than the rows need: one block covers up to 16 * cap rows.)
  const int gx = a.n_tiles / a.NT;
  const int cap = min(fit, max(1, (a.M + 15) / 16));
  int MT = cap;
  for (int mt = 1; mt < cap; ++mt)
    if ((long)gx * a.S * ((a.M + 16 * mt - 1) / (16 * mt)) <= kGemmPersistentWgs) { MT = mt; break; }
  if (EPI == EPI_RESID && a.NT * MT * 16 * 16 > 2 * kGemmThreads) return hipErrorInvalidValue;
  if (EPI == EPI_LOGITS && a.NT > 4) return hipErrorInvalidValue;   // the top-2 scan holds 2 * NT columns per lane
  if (EPI == EPI_PARTIAL && (a.S < 2 || a.S > 8)) return hipErrorInvalidValue;
  if (MT == 1) return launch_gemm_mt<T, EPI, 1>(a, st);
  if (MT == 2) return launch_gemm_mt<T, EPI, 2>(a, st);
  return launch_gemm_mt<T, EPI, 3>(a, st);
}

template <typename T>
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return a.NT == 1 ? launch_gemm_epi<T, EPI_QKV>(a, st) : hipErrorInvalidValue;
    case EPI_RESID: return launch_gemm_epi<T, EPI_RESID>(a, st);
    case EPI_PARTIAL: return launch_gemm_epi<T, EPI_PARTIAL>(a, st);
    case EPI_SWIGLU: return launch_gemm_epi<T, EPI_SWIGLU>(a, st);
    default: return launch_gemm_epi<T, EPI_LOGITS>(a, st);
  }
}
template hipError_t launch_gemm<bf16_t>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs&, int, hipStream_t);

template <int EPI, int RT, int CT, int NS, bool EXACT, int WC = 2>
static hipError_t launch_gemm_big_cfg(const GemmArgs& a, hipStream_t st) {
  constexpr int NF = WC * CT + 2 * RT;
  const dim3 grid(a.n_tiles / (WC * CT), (a.M + 32 * RT - 1) / (32 * RT));
  const int shm = NS * NF * 1024 + 32 * RT * 4;
  SSB_LAUNCH((k_gemm_big<EPI, RT, CT, NS, EXACT, WC>), grid, dim3(2 * WC * kWave), shm, st, a);
  return hipGetLastError();
}

template <int EPI, bool EXACT>
static hipError_t launch_gemm_big_epi(const GemmArgs& a, hipStream_t st) {
  if constexpr (EPI == EPI_LOGITS) {
    // 128 x 128 blocks: each wave's 64 columns are one LM head group
    return a.n_tiles % 8 == 0 ? launch_gemm_big_cfg<EPI, 4, 4, 3, true>(a, st) : hipErrorInvalidValue;
  } else {
    // the largest tile that still gives about one workgroup per CU; non-exact (prefill) GEMMs wide
    // enough take 128 x 256 blocks of eight waves at two workgroups per CU (JIT fragment reads;
    // against four waves of 64 x 128: 41.0 -> 38.2 us for the 1088-row gate|up)
    const int rb4 = (a.M + 127) / 128;
    // (LDS: 3 steps of 16 KiB, 4 of 12 KiB, 6 of 8 KiB: two or three workgroups per CU; deeper
    // pipelines with one workgroup per CU measured slower)
    if constexpr (!EXACT && EPI == EPI_SWIGLU) {   // (the QKV epilogue would spill at 128 VGPRs)
      if (a.n_tiles % 16 == 0 && (a.n_tiles / 16) * rb4 >= 240) return launch_gemm_big_cfg<EPI, 4, 4, 3, false, 4>(a, st);
    }
    if (a.n_tiles % 8 == 0 && (a.n_tiles / 8) * rb4 >= 240) return launch_gemm_big_cfg<EPI, 4, 4, 3, EXACT>(a, st);
    if (a.n_tiles % 4 == 0 && (a.n_tiles / 4) * rb4 >= 240) return launch_gemm_big_cfg<EPI, 4, 2, 4, EXACT>(a, st);
    // (the 4096-deep down projection keeps eight steps in flight: 33.6 -> 31.5 us in a prefill)
    if constexpr (!EXACT) {
      if (a.n_tiles % 4 == 0 && a.K >= 4096) return launch_gemm_big_cfg<EPI, 2, 2, 8, false>(a, st);
    }
    if (a.n_tiles % 4 == 0) return launch_gemm_big_cfg<EPI, 2, 2, 6, EXACT>(a, st);
    return hipErrorInvalidValue;
  }
}

// Large-tile GEMM (bf16, M >= 1): epilogues QKV, RESID (no K split) and SWIGLU.  exact: the
// arithmetic of k_gemm for the same plan (a.S == 1, a.KSL slices), for tall decode forwards;
// it also has the LM head's records (LOGITS, without the softmax sums).
hipError_t launch_gemm_big(const GemmArgs& a, int epi, bool exact, hipStream_t st) {
  if (a.M < 1 || a.K % Ty<bf16_t>::kStepK != 0 || a.n_tiles % 4 != 0) return hipErrorInvalidValue;
  if ((epi == EPI_QKV || epi == EPI_SWIGLU) && (a.n_ssq % 2 != 0 || a.n_ssq < 2)) return hipErrorInvalidValue;
  if (exact) {
    const int ksteps = a.K / Ty<bf16_t>::kStepK;
    const int G = a.n_ssq / 4;
    if (a.S != 1 || a.KSL < 1 || ksteps % a.KSL != 0) return hipErrorInvalidValue;
    if ((epi == EPI_QKV || epi == EPI_SWIGLU) && (a.n_ssq % 4 != 0 || G > 64 || (G & (G - 1)) != 0))
      return hipErrorInvalidValue;
    switch (epi) {
      case EPI_QKV: return launch_gemm_big_epi<EPI_QKV, true>(a, st);
      case EPI_RESID: return launch_gemm_big_epi<EPI_RESID, true>(a, st);
      case EPI_SWIGLU: return launch_gemm_big_epi<EPI_SWIGLU, true>(a, st);
      case EPI_LOGITS:   // records of 4-tile groups only (no softmax sums)
        return a.am_s || a.NT != 4 ? hipErrorInvalidValue : launch_gemm_big_epi<EPI_LOGITS, true>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_QKV: return launch_gemm_big_epi<EPI_QKV, false>(a, st);
    case EPI_RESID: return launch_gemm_big_epi<EPI_RESID, false>(a, st);
    case EPI_SWIGLU: return launch_gemm_big_epi<EPI_SWIGLU, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}


template <typename T>
hipError_t launch_resid_reduce(const GemmArgs& a, hipStream_t st) {
  if (a.S < 1 || a.S > 8 || a.hidden % 64 != 0) return hipErrorInvalidValue;
  SSB_LAUNCH(k_resid_reduce<T>, dim3(a.M, a.hidden / 64), dim3(64), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_resid_reduce<bf16_t>(const GemmArgs&, hipStream_t);
template hipError_t launch_resid_reduce<float>(const GemmArgs&, hipStream_t);

hipError_t launch_argmax(const float* v1, const int32_t* i1, const float* v2, const float* gs, float sc, int n_groups,
                         int ld, int M, int32_t* tok, float* top1, float* top2, float* zs, hipStream_t st,
                         ProfStamp* stamp, const int* err) {
  if (gs && !zs) return hipErrorInvalidValue;
  SSB_LAUNCH(k_argmax, dim3(M), dim3(kThreads), 0, st, v1, i1, v2, gs, sc, n_groups, ld, tok, top1, top2, zs, stamp,
             err);
  return hipGetLastError();
}

// Rows j = 0..rows_per_req-1 of every request (row row0[r] + j of the launch), each drawn
// with u[r][j]; gcols (columns per LM-head group) must be <= 64.
hipError_t launch_sample_rows(const SampleArgs& a, int rows_per_req, int n_req, hipStream_t st) {
  if (a.gcols < 1 || a.gcols > kWave || rows_per_req < 1 || n_req < 1 || n_req > kMaxReq) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sample_rows, dim3(rows_per_req, n_req), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_accept_sample(const AcceptSampleArgs& a, int n_req, hipStream_t st) {
  if (n_req < 1 || n_req > kMaxReq) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept_sample, dim3(n_req), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn(const AttnArgs& a, int n_chunk_slots, int head_dim, hipStream_t st) {
  if (a.n_heads / a.n_kv > kAttnThreads / kWave) return hipErrorInvalidValue;
  if (!a.fold && n_chunk_slots > a.max_chunks) return hipErrorInvalidValue;
  dim3 grid(a.fold ? 1 : n_chunk_slots, a.n_kv, a.tasks.n * (kTaskRows / 16));
  // folded rows: fold_streams<T>() chunk streams per workgroup
  if (head_dim == 64) {
    if (a.fold) SSB_LAUNCH((k_attn<T, 64, true>), grid, dim3(fold_streams<T>() * kAttnThreads), 0, st, a);
    else SSB_LAUNCH((k_attn<T, 64, false>), grid, dim3(kAttnThreads), 0, st, a);
  } else {
    if (a.fold) SSB_LAUNCH((k_attn<T, 32, true>), grid, dim3(fold_streams<T>() * kAttnThreads), 0, st, a);
    else SSB_LAUNCH((k_attn<T, 32, false>), grid, dim3(kAttnThreads), 0, st, a);
  }
  return hipGetLastError();
}
template hipError_t launch_attn<bf16_t>(const AttnArgs&, int, int, hipStream_t);
template hipError_t launch_attn<float>(const AttnArgs&, int, int, hipStream_t);

template <typename T>
hipError_t launch_attn_combine(const float* part, int max_chunks, int n_slots, int n_heads, int head_dim,
                               const int32_t* row_lim, int M, void* out, int out_ld, hipStream_t st,
                               ProfStamp* stamp) {
  if (n_slots < 1 || n_slots > max_chunks) return hipErrorInvalidValue;
  // one single-wave workgroup per (row, head): spread over every CU (4-wave workgroups on half
  // the CUs measured 0.2-0.3 us slower per launch, 2-wave ones slower still)
  const int blocks = M * n_heads;
  if (head_dim == 64)
    SSB_LAUNCH((k_attn_combine<T, 64>), dim3(blocks), dim3(kWave), 0, st, part, max_chunks, n_slots,
                       n_heads, row_lim, M, out, out_ld, stamp);
  else
    SSB_LAUNCH((k_attn_combine<T, 32>), dim3(blocks), dim3(kWave), 0, st, part, max_chunks, n_slots,
                       n_heads, row_lim, M, out, out_ld, stamp);
  return hipGetLastError();
}
template hipError_t launch_attn_combine<bf16_t>(const float*, int, int, int, int, const int32_t*, int, void*, int,
                                                hipStream_t, ProfStamp*);
template hipError_t launch_attn_combine<float>(const float*, int, int, int, int, const int32_t*, int, void*, int,
                                               hipStream_t, ProfStamp*);

template <typename T>
hipError_t launch_poison_kv(const ReqArgs* req, int R, const int32_t* acc, int acc_stride, int lo_abs, int hi_abs,
                            void* kv_pool, int n_layers, int n_pages, int n_kv, int hd, hipStream_t st) {
  hipLaunchKernelGGL((k_poison_kv<T>), dim3(R * n_layers), dim3(256), 0, st, req, acc, acc_stride, lo_abs, hi_abs,
                     kv_pool, n_layers, n_pages, n_kv, hd);
  return hipGetLastError();
}
template hipError_t launch_poison_kv<bf16_t>(const ReqArgs*, int, const int32_t*, int, int, int, void*, int, int, int,
                                             int, hipStream_t);
template hipError_t launch_poison_kv<float>(const ReqArgs*, int, const int32_t*, int, int, int, void*, int, int, int,
                                            int, hipStream_t);

hipError_t launch_accept(const int32_t* row_tok, const int32_t* am, const ReqArgs* ra, int n_req, int eos_id,
                         int32_t* out, int out_stride, hipStream_t st, const int* err, ProfStamp* stamp) {
  SSB_LAUNCH(k_accept, dim3(n_req), dim3(64), 0, st, row_tok, am, ra, eos_id, out, out_stride, err, stamp);
  return hipGetLastError();
}

// The request state's B must be <= 64 (one lane per block position) and rec_stride >= 4 + 4 * B;
// both are checked by the engine before the request state is uploaded.
hipError_t launch_dd_init(const ReqArgs* ra, int n_req, int mask_id, int32_t* rec, int rec_stride, hipStream_t st) {
  if (n_req < 1 || n_req > kMaxReq || rec_stride < 4 + 4 * kWave) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dd_init, dim3(n_req), dim3(kWave), 0, st, ra, mask_id, rec, rec_stride);
  return hipGetLastError();
}

hipError_t launch_dd_select(const int32_t* am, const float* zs, const ReqArgs* ra, int n_req, int mask_id,
                            int vocab, int32_t* rec, int rec_stride, hipStream_t st) {
  if (n_req < 1 || n_req > kMaxReq || rec_stride < 4 + 4 * kWave) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dd_select, dim3(n_req), dim3(kWave), 0, st, am, zs, ra, mask_id, vocab, rec, rec_stride);
  return hipGetLastError();
}

// One launch per decode layer: kTailWgs workgroups of nine waves, one per CU (the slab of the down
// stage keeps a second one off a CU).  Shapes must be those the fused kernel is written for; anything else is
// hipErrorInvalidValue and the engine runs the three GEMM launches instead.
int layer_tail_lds(int n_ssq) {
  const int o = gemm_lds(1, 8 * 4 * 32 * 2, 1, 8, n_ssq, EPI_RESID).total;
  const int g = gemm_lds(3, 4 * 8 * 32 * 2, 2, 4, n_ssq, EPI_SWIGLU).total;
  const int d = gemm_lds(1, 8 * 16 * 32 * 2, 1, 8, n_ssq, EPI_RESID).total;
  return max(o, max(g, d));
}

hipError_t launch_layer_tail(const TailArgs& a, hipStream_t st) {
  const int M = a.o.M, nrb = (M + 15) / 16;
  const bool ok = M >= 1 && M <= 48 && a.gu.M == M && a.d.M == M && a.o.S == 1 && a.d.S == 1 &&
                  a.o.NT == 1 && a.o.KSL == 8 && a.o.K == 8 * 4 * 32 &&
                  a.gu.NT == 2 && a.gu.KSL == 4 && a.gu.K == 4 * 8 * 32 && a.gu.n_tiles == 2 * kTailWgs &&
                  a.d.NT == 1 && a.d.KSL == 8 && a.d.K == 8 * 16 * 32 &&
                  a.o.n_tiles * nrb <= kTailWgs && a.d.n_tiles * nrb <= kTailWgs && a.o.n_tiles == a.d.n_tiles &&
                  a.o.hidden == a.o.n_tiles * 16 && a.gu.n_ssq == a.o.hidden / 16 && a.gu.n_ssq % 4 == 0 &&
                  a.gu.n_ssq / 4 <= 64 && ((a.gu.n_ssq / 4) & (a.gu.n_ssq / 4 - 1)) == 0 && a.sync && a.err;
  if (!ok) return hipErrorInvalidValue;
  const int shm = layer_tail_lds(a.gu.n_ssq);
  if (shm + 4096 > 160 * 1024) return hipErrorInvalidValue;   // the kernel's static arrays take < 4 KiB
  SSB_LAUNCH((k_layer_tail<4, 8, 16>), dim3(kTailWgs), dim3(kTailThreads), shm, st, a);
  return hipGetLastError();
}

}  // namespace ssb
