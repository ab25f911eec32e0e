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

namespace ssb {

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
                       const T* src2, int n0, int n1, int hd) {
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
      tok = j == 0 ? ra.x0[r] : a.mask_id;
      pos = p + j;
      lim = j == 0 ? p : p + ra.B;
    } else {
      // verify window [a0, d1..dB] at p+1..p+B+1, causal; row j of the draft
      // predicted a0 (j = 0) or d_j
      pos = p + 1 + j;
      lim = pos;
      tok = a.am_prev[m];
      if (j >= 1) {
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
  int tok, pos, lim, req;
  window_row(a, m, tok, pos, lim, req);
  if (g == 0 && t == 0) {
    a.row_tok[m] = tok; a.row_pos[m] = pos; a.row_lim[m] = lim; a.row_req[m] = req;
  }
  const int col = g * 64 + t;
  const T* src = tok >= 0 ? reinterpret_cast<const T*>(a.embed) + (size_t)tok * a.hidden
                          : reinterpret_cast<const T*>(a.prefix) + (size_t)pos * a.hidden;
  const float v = Ty<T>::to_f(src[col]);
  a.h[(size_t)m * a.hidden + col] = v;
  reinterpret_cast<T*>(a.xg)[(size_t)m * a.hidden + col] = Ty<T>::from_f(v * a.gain[col]);
  float s = v * v;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
  if (t % 16 == 0) a.ssq[(size_t)(col / 16) * a.ssq_ld + m] = s;
}

// ---------------------------------------------------------------------------
// GEMM with fused epilogues:  out[m][n] = sum_k X[m][k] W[n][k].
// Grid (n_tiles, m_blocks); a workgroup owns one 16-column tile for 16*MT
// rows and the full K.  Wave w of W = ksteps/KPW waves reduces K steps
// [w*KPW, (w+1)*KPW) with an MFMA chain in K order after loading all of its
// weight and activation fragments at once; the W partial tiles are then
// added in wave order through LDS.  The decomposition depends only on K, so
// a row's value never depends on M.
// RMSNorm inputs arrive as X = h * gain (in T) and each output row is scaled
// by 1/rms(h), rms from the per-16-column sums of squares added in column
// order (review section 3.1: both modes share these layers).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <typename T, int MT, int EPI, int KPW>
__global__ __launch_bounds__(1024) void k_gemm(GemmArgs a) {
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int MB = MT * 16;
  constexpr bool NORM = (EPI != EPI_RESID);
  extern __shared__ __align__(16) unsigned char smem[];
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);          // [W][MT][64]
  __shared__ float ctile[MB][17];
  __shared__ float s_inv[MB];
  __shared__ float s_ssq[kMaxNormParts * MB];

  const int tile = blockIdx.x;
  const int m_base = blockIdx.y * MB;
  const int W = blockDim.x / kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ksteps = a.K / KS;
  const int k0 = wave * KPW;

  // weights of this wave (the HBM-latency-critical loads) go out first, all at once
  uint4 wf[KPW];
  const uint4* wp = a.W + ((size_t)tile * ksteps + k0) * kWave + lane;
#pragma unroll
  for (int s = 0; s < KPW; ++s) wf[s] = wp[(size_t)s * kWave];
  // row-norm statistics: every thread helps load the per-16-column partials
  if constexpr (NORM) {
    for (int e = threadIdx.x; e < a.n_ssq * MB; e += blockDim.x) {
      const int gi = e / MB, r = e % MB;
      const int m = m_base + r;
      s_ssq[gi * MB + r] = m < a.M ? a.ssq[(size_t)gi * a.ssq_ld + m] : 0.f;
    }
  }
  // activation fragments in phases of up to 4 K steps (bounded register use)
  constexpr int PH = KPW < 4 ? KPW : 4;
  const T* xb = reinterpret_cast<const T*>(a.x);
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p0 = 0; p0 < KPW; p0 += PH) {
    uint4 xf[PH][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = m_base + mt * 16 + lane % 16;
#pragma unroll
      for (int s = 0; s < PH; ++s) {
        xf[s][mt] = make_uint4(0, 0, 0, 0);
        if (row < a.M)
          xf[s][mt] = *reinterpret_cast<const uint4*>(xb + (size_t)row * a.ldx + (k0 + p0 + s) * KS +
                                                      PER * (lane / 16));
      }
    }
#pragma unroll
    for (int s = 0; s < PH; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mma_step(acc[mt], wf[p0 + s], xf[s][mt], T());
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * kWave + lane] = acc[mt];
  __syncthreads();
  if constexpr (NORM) {
    for (int r = threadIdx.x; r < MB; r += blockDim.x) {
      float s = 0.f;
      for (int gi = 0; gi < a.n_ssq; ++gi) s += s_ssq[gi * MB + r];
      s_inv[r] = 1.0f / sqrtf(s / (float)a.hidden + a.eps);
    }
  }
  for (int e = threadIdx.x; e < MT * kWave * 4; e += blockDim.x) {
    const int mt = e / (kWave * 4), l = (e / 4) % kWave, i = e % 4;
    float s = 0.f;
    for (int w = 0; w < W; ++w) s += red[(w * MT + mt) * kWave + l][i];
    ctile[mt * 16 + l % 16][4 * (l / 16) + i] = s;     // [row][tile column]
  }
  __syncthreads();

  if constexpr (EPI == EPI_QKV) {
    const int hd = a.head_dim, half = hd / 2, tph = hd / 16;
    const int hh = tile / tph, jj = tile % tph;
    const int kind = hh < a.n_heads ? 0 : (hh < a.n_heads + a.n_kv ? 1 : 2);   // q, k, v
    const int head = kind == 0 ? hh : (kind == 1 ? hh - a.n_heads : hh - a.n_heads - a.n_kv);
    for (int e = threadIdx.x; e < MB * 8; e += blockDim.x) {
      const int r = e / 8, c = e % 8;
      const int m = m_base + r;
      if (m >= a.M) continue;
      const float inv = s_inv[r];
      float x1 = ctile[r][c] * inv, x2 = ctile[r][c + 8] * inv;
      const int i = 8 * jj + c;                 // rotary pair (i, i + hd/2)
      const int pos = a.row_pos[m];
      if (kind != 2) {
        const float2 cs = a.rope[(size_t)pos * half + i];
        const float o1 = x1 * cs.x - x2 * cs.y;
        const float o2 = x2 * cs.x + x1 * cs.y;
        x1 = o1; x2 = o2;
      }
      T* dst;
      if (kind == 0) {
        dst = reinterpret_cast<T*>(a.q) + (size_t)m * a.q_ld + head * hd;
      } else {
        const int32_t* pt = a.req->pt[a.row_req[m]];
        const int page = pt[pos / kPage], slot = pos % kPage;
        const size_t base = (((size_t)a.layer * a.n_pages + page) * 2 + (kind - 1)) * a.n_kv + head;
        dst = reinterpret_cast<T*>(a.kv_pool) + (base * kPage + slot) * hd;
      }
      dst[i] = Ty<T>::from_f(x1);
      dst[i + half] = Ty<T>::from_f(x2);
    }
  } else if constexpr (EPI == EPI_RESID) {
    for (int e = threadIdx.x; e < MB * 16; e += blockDim.x) {
      const int r = e / 16, n = e % 16;
      const int m = m_base + r;
      if (m >= a.M) continue;
      const int col = tile * 16 + n;
      float* hp = a.h + (size_t)m * a.hidden + col;
      const float v = *hp + ctile[r][n];
      *hp = v;
      reinterpret_cast<T*>(a.xg_out)[(size_t)m * a.hidden + col] = Ty<T>::from_f(v * a.gain_next[col]);
      ctile[r][n] = v;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < MB; r += blockDim.x) {
      const int m = m_base + r;
      if (m >= a.M) continue;
      float s = 0.f;
      for (int n = 0; n < 16; ++n) s += ctile[r][n] * ctile[r][n];
      a.ssq_out[(size_t)tile * a.ssq_ld + m] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int e = threadIdx.x; e < MB * 8; e += blockDim.x) {
      const int r = e / 8, c = e % 8;
      const int m = m_base + r;
      if (m >= a.M) continue;
      const float g = ctile[r][c] * s_inv[r];
      const float u = ctile[r][c + 8] * s_inv[r];
      reinterpret_cast<T*>(a.act)[(size_t)m * a.act_ld + tile * 8 + c] = Ty<T>::from_f(silu_f(g) * u);
    }
  } else {  // EPI_LOGITS
    for (int e = threadIdx.x; e < MB * 16; e += blockDim.x) {
      const int r = e / 16, n = e % 16;
      const int m = m_base + r;
      const float z = ctile[r][n] * s_inv[r];
      ctile[r][n] = z;
      const int col = tile * 16 + n;
      if (a.logits && m < a.M && col < a.vocab) a.logits[(size_t)m * a.vocab + col] = z;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < MB; r += blockDim.x) {
      const int m = m_base + r;
      if (m >= a.M) continue;
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7fffffff;
      bool nan = false;
      for (int n = 0; n < 16; ++n) {
        const int col = tile * 16 + n;
        if (col >= a.vocab || col == a.mask_id) continue;
        const float z = ctile[r][n];
        if (z != z) { nan = true; continue; }
        if (z > v1) { v2 = v1; v1 = z; i1 = col; }
        else if (z > v2) { v2 = z; }
      }
      if (nan) { v1 = NAN; v2 = NAN; i1 = -1; }
      a.am_v1[(size_t)tile * a.am_ld + m] = v1;
      a.am_i1[(size_t)tile * a.am_ld + m] = i1;
      a.am_v2[(size_t)tile * a.am_ld + m] = v2;
    }
  }
}

// ---------------------------------------------------------------------------
// Greedy argmax over the vocabulary without [M], lowest id on ties, with the
// runner-up value (GravityOCR review, section 2 "Speculative Decoding":
// greedy top-1 verification).  Merging (top1 value, top1 id, top2 value)
// records is associative and commutative, so any reduction tree gives the
// same bits.  A NaN anywhere makes the row's record NaN.
// ---------------------------------------------------------------------------
struct Top2 { float v1; int i1; float v2; };

__device__ __forceinline__ Top2 merge_top2(Top2 a, Top2 b) {
  if (a.i1 == -1 || b.i1 == -1) return Top2{NAN, -1, NAN};
  const bool bw = b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1);
  Top2 r;
  if (bw) { r.v1 = b.v1; r.i1 = b.i1; r.v2 = fmaxf(a.v1, b.v2); }
  else { r.v1 = a.v1; r.i1 = a.i1; r.v2 = fmaxf(a.v2, b.v1); }
  return r;
}

__global__ __launch_bounds__(kThreads) void k_argmax(const float* v1, const int32_t* i1, const float* v2,
                                                    int n_groups, int ld, int32_t* tok, float* top1,
                                                    float* top2) {
  __shared__ Top2 sh[kThreads];
  const int m = blockIdx.x;
  constexpr int BATCH = 16;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  for (int g0 = threadIdx.x; g0 < n_groups; g0 += BATCH * kThreads) {
    Top2 rec[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int g = g0 + b * kThreads;
      rec[b] = Top2{-INFINITY, 0x7fffffff, -INFINITY};
      if (g < n_groups) rec[b] = Top2{v1[(size_t)g * ld + m], i1[(size_t)g * ld + m], v2[(size_t)g * ld + m]};
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) t = merge_top2(t, rec[b]);
  }
  sh[threadIdx.x] = t;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] = merge_top2(sh[threadIdx.x], sh[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    tok[m] = sh[0].i1;
    top1[m] = sh[0].v1;
    top2[m] = sh[0].v2;
  }
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
// Online-softmax merge of a running (m, l, o) with a chunk record (mc, lc, oc):
// m' = max(m, mc), l' = l e^(m-m') + lc e^(mc-m'), o' likewise.
__device__ __forceinline__ void fold_coef(float m, float mc, float& mn, float& al, float& be) {
  mn = fmaxf(m, mc);
  al = expf(m - mn);
  be = expf(mc - mn);
}
__device__ __forceinline__ float fold_val(float v, float al, float vc, float be) {
  return __fadd_rn(__fmul_rn(v, al), __fmul_rn(vc, be));
}

template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int DT = HD / 16;
  constexpr int QKS = HD / KS;             // steps of S^T over the head dimension
  constexpr int KT = kKeyChunk / 16;       // key tiles per chunk
  constexpr int PVS = kKeyChunk / KS;      // steps of P V over keys
  constexpr int KSTR = HD * (int)sizeof(T) + 16;              // K rows [key][d]
  constexpr int VSTR = kKeyChunk * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);   // V^T rows [d][key]
  constexpr int MT = kTaskRows / 16;
  constexpr int REC = HD + 4;
  constexpr int MAXU = 3;                  // units per wave: ceil(4 heads * 3 tiles / 4 waves)
  constexpr int FPK = HD / PER;            // 16-byte fragments per key row
  constexpr int KVF = 2 * kKeyChunk * FPK / kThreads;   // fragments per thread
  __shared__ __align__(16) unsigned char ks[kKeyChunk * KSTR];
  __shared__ __align__(16) unsigned char vts[HD * VSTR];
  __shared__ int s_lim[kTaskRows];

  const AttnTask task = a.tasks.t[blockIdx.z];
  const int g = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n_rep = a.n_heads / a.n_kv;
  const int32_t* pt = a.req->pt[task.req];
  const int n_units = n_rep * MT;

  if (threadIdx.x < kTaskRows)
    s_lim[threadIdx.x] = threadIdx.x < task.nrows ? a.row_lim[task.row0 + threadIdx.x] : -1;
  // largest visibility limit of the task's rows
  const int maxlim = task.lim_mode == 0 ? task.max_lim : a.req->p[task.req] + a.req->B + (task.lim_mode == 2 ? 1 : 0);
  int cbeg, cend;
  if (a.fold) { cbeg = 0; cend = maxlim / kKeyChunk + 1; }
  else {
    cbeg = blockIdx.x; cend = cbeg + 1;
    if (cbeg * kKeyChunk > maxlim) return;
  }

  // query fragments of this wave's units (B operand of S^T): issued first
  uint4 qf[MAXU][QKS];
#pragma unroll
  for (int ui = 0; ui < MAXU; ++ui) {
    const int u = wave + 4 * ui;
    const int hl = u / MT, mt = u % MT;
    const int row_local = mt * 16 + lane % 16;
#pragma unroll
    for (int st = 0; st < QKS; ++st) {
      qf[ui][st] = make_uint4(0, 0, 0, 0);
      if (u < n_units && row_local < task.nrows)
        qf[ui][st] = *reinterpret_cast<const uint4*>(
            reinterpret_cast<const T*>(a.q) + (size_t)(task.row0 + row_local) * a.q_ld + (g * n_rep + hl) * HD +
            st * KS + PER * (lane / 16));
    }
  }

  float run_m[MAXU], run_l[MAXU];
  f32x4_t run_o[MAXU][DT];
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    run_m[u] = -INFINITY; run_l[u] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) run_o[u][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int c = cbeg; c < cend; ++c) {
    // K and V of keys [c*64, c*64+64) that any row of the task may see
    uint4 kvv[KVF];
#pragma unroll
    for (int q = 0; q < KVF; ++q) {
      const int f = threadIdx.x + q * kThreads;
      const int kv = f / (kKeyChunk * FPK);
      const int rem = f % (kKeyChunk * FPK);
      const int key = c * kKeyChunk + rem / FPK;
      kvv[q] = make_uint4(0, 0, 0, 0);
      if (key <= maxlim) {
        const int page = pt[key / kPage], slot = key % kPage;
        const size_t base = (((size_t)a.layer * a.n_pages + page) * 2 + kv) * a.n_kv + g;
        kvv[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.kv_pool) +
                                                 (base * kPage + slot) * HD + (rem % FPK) * PER);
      }
    }
#pragma unroll
    for (int q = 0; q < KVF; ++q) {
      const int f = threadIdx.x + q * kThreads;
      const int kv = f / (kKeyChunk * FPK);
      const int rem = f % (kKeyChunk * FPK);
      const int kk = rem / FPK, d0 = (rem % FPK) * PER;
      if (kv == 0) {
        *reinterpret_cast<uint4*>(ks + kk * KSTR + d0 * (int)sizeof(T)) = kvv[q];
      } else {
        const T* vals = reinterpret_cast<const T*>(&kvv[q]);
#pragma unroll
        for (int i = 0; i < PER; ++i) *reinterpret_cast<T*>(vts + (d0 + i) * VSTR + kk * (int)sizeof(T)) = vals[i];
      }
    }
    __syncthreads();

#pragma unroll
    for (int ui = 0; ui < MAXU; ++ui) {
      const int u = wave + 4 * ui;
      if (u >= n_units) break;
      const int hl = u / MT, mt = u % MT;
      if (mt * 16 >= task.nrows) continue;
      const int head = g * n_rep + hl;
      const int row_local = mt * 16 + lane % 16;
      // S^T tiles: element i of tile kt = score of key kt*16 + 4*(lane/16) + i for row_local
      f32x4_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QKS; ++st) {
          const uint4 kf = *reinterpret_cast<const uint4*>(
              ks + (kt * 16 + lane % 16) * KSTR + (st * KS + PER * (lane / 16)) * (int)sizeof(T));
          mma_step(s[kt], kf, qf[ui][st], T());
        }
      }
      const int lim = s_lim[row_local];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = c * kKeyChunk + kt * 16 + 4 * (lane / 16) + i;
          const float z = key <= lim ? s[kt][i] * a.scale : -INFINITY;
          s[kt][i] = z;
          mx = fmaxf(mx, z);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = (s[kt][i] == -INFINITY) ? 0.f : expf(s[kt][i] - mx);
          s[kt][i] = p;
          lsum += p;
        }
      lsum = lsum + __shfl_xor(lsum, 16);
      lsum = lsum + __shfl_xor(lsum, 32);
      // o^T = V^T P^T ; lane supplies keys pi(lane, j) for P^T and V^T alike
      f32x4_t o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const unsigned char* vrow = vts + (dt * 16 + lane % 16) * VSTR;
#pragma unroll
        for (int st = 0; st < PVS; ++st) {
          uint4 pf, vf;
          if constexpr (sizeof(T) == 2) {
            // keys 32st + 4(l/16) + {0..3} from tile 2st, then the same +16 from tile 2st+1
            const f32x4_t p0 = s[2 * st], p1 = s[2 * st + 1];
            pf.x = (uint32_t)f2bf(p0[0]) | ((uint32_t)f2bf(p0[1]) << 16);
            pf.y = (uint32_t)f2bf(p0[2]) | ((uint32_t)f2bf(p0[3]) << 16);
            pf.z = (uint32_t)f2bf(p1[0]) | ((uint32_t)f2bf(p1[1]) << 16);
            pf.w = (uint32_t)f2bf(p1[2]) | ((uint32_t)f2bf(p1[3]) << 16);
            const uint2 va = *reinterpret_cast<const uint2*>(vrow + (32 * st + 4 * (lane / 16)) * 2);
            const uint2 vb = *reinterpret_cast<const uint2*>(vrow + (32 * st + 16 + 4 * (lane / 16)) * 2);
            vf = make_uint4(va.x, va.y, vb.x, vb.y);
          } else {
            const f32x4_t p0 = s[st];
            pf = make_uint4(__float_as_uint(p0[0]), __float_as_uint(p0[1]), __float_as_uint(p0[2]),
                            __float_as_uint(p0[3]));
            vf = *reinterpret_cast<const uint4*>(vrow + (16 * st + 4 * (lane / 16)) * 4);
          }
          mma_step(o[dt], vf, pf, T());
        }
      }
      // o[dt][i] = o_c[d = dt*16 + 4*(lane/16) + i] of row_local
      if (a.fold) {
        float mn, al, be;
        fold_coef(run_m[ui], mx, mn, al, be);
        run_l[ui] = fold_val(run_l[ui], al, lsum, be);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) run_o[ui][dt][i] = fold_val(run_o[ui][dt][i], al, o[dt][i], be);
        run_m[ui] = mn;
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

  if (a.fold) {
#pragma unroll
    for (int ui = 0; ui < MAXU; ++ui) {
      const int u = wave + 4 * ui;
      if (u >= n_units) break;
      const int hl = u / MT, mt = u % MT;
      const int row_local = mt * 16 + lane % 16;
      if (row_local >= task.nrows) continue;
      const int head = g * n_rep + hl;
      T* dst = reinterpret_cast<T*>(a.out) + (size_t)(task.row0 + row_local) * a.out_ld + head * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[dt * 16 + 4 * (lane / 16) + i] = Ty<T>::from_f(run_o[ui][dt][i] / run_l[ui]);
    }
  }
}

// Combine the per-chunk records of each (row, head) in chunk order.
// One wave per (row, head); lane d holds output dimension d.  Records are
// loaded 32 chunks at a time before folding.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_combine(const float* part, int max_chunks, int n_heads,
                                                          const int32_t* row_lim, int M, void* out,
                                                          int out_ld) {
  constexpr int REC = HD + 4;
  constexpr int BATCH = 32;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= M * n_heads) return;
  const int row = idx / n_heads, head = idx % n_heads;
  const int nch = row_lim[row] / kKeyChunk + 1;
  const float* rec = part + ((size_t)row * n_heads + head) * max_chunks * REC;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int c0 = 0; c0 < nch; c0 += BATCH) {
    float mc[BATCH], lc[BATCH], oc[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = c0 + b;
      mc[b] = -INFINITY; lc[b] = 0.f; oc[b] = 0.f;
      if (c < nch) {
        const float2 ml = *reinterpret_cast<const float2*>(rec + c * REC + HD);
        mc[b] = ml.x; lc[b] = ml.y;
        if (lane < HD) oc[b] = rec[c * REC + lane];
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (c0 + b < nch) {
        float mn, al, be;
        fold_coef(m, mc[b], mn, al, be);
        l = fold_val(l, al, lc[b], be);
        o = fold_val(o, al, oc[b], be);
        m = mn;
      }
    }
  }
  if (lane < HD) reinterpret_cast<T*>(out)[(size_t)row * out_ld + head * HD + lane] = Ty<T>::from_f(o / l);
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
                                               int eos_id, int32_t* out, int out_stride) {
  const ReqArgs& ra = *rap;
  const int r = blockIdx.x, j = threadIdx.x;
  const int B = ra.B, row0 = ra.row0[r];
  const bool mismatch = j < B && row_tok[row0 + 1 + j] != am[row0 + j];
  const unsigned long long bal = __ballot(mismatch);
  const int A = bal ? __builtin_ctzll(bal) : B;
  int32_t* o = out + (size_t)r * out_stride;
  // candidate commit list: k = 0 -> a0, k >= 1 -> a_k = am[row0 + k - 1]
  const int ncand = A + 2;
  int eos_at = ncand;
  for (int k = 0; k < ncand; ++k) {
    const int tk = k == 0 ? row_tok[row0] : am[row0 + k - 1];
    if (tk == eos_id) { eos_at = k; break; }
  }
  int n = min(ncand, eos_at + 1);
  n = min(n, ra.max_commit[r]);
  for (int k = j; k < n; k += 64) o[4 + k] = k == 0 ? row_tok[row0] : am[row0 + k - 1];
  if (j == 0) {
    o[0] = A;
    o[1] = n;
    o[2] = am[row0 + A];
    o[3] = (eos_at < ncand && eos_at < n) ? 1 : 0;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (C++ linkage, used by the engine).
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_pack(uint4* dst, int n_tiles, int K, int mode, const void* s0, const void* s1,
                       const void* s2, int n0, int n1, int hd, hipStream_t st) {
  hipLaunchKernelGGL(k_pack<T>, dim3(1024), dim3(256), 0, st, dst, n_tiles, K, mode,
                     (const T*)s0, (const T*)s1, (const T*)s2, n0, n1, hd);
  return hipGetLastError();
}
template hipError_t launch_pack<bf16_t>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                        int, int, hipStream_t);
template hipError_t launch_pack<float>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                       int, int, hipStream_t);

template <typename T>
hipError_t launch_prep(const PrepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_prep_embed<T>, dim3(a.M, a.hidden / 64), dim3(64), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_prep<bf16_t>(const PrepArgs&, hipStream_t);
template hipError_t launch_prep<float>(const PrepArgs&, hipStream_t);

template <typename T, int EPI, int KPW>
static hipError_t launch_gemm_kpw(const GemmArgs& a, int MT, hipStream_t st) {
  const int ksteps = a.K / Ty<T>::kStepK;
  const int W = ksteps / KPW;
  const int m_blocks = (a.M + 16 * MT - 1) / (16 * MT);
  const dim3 grid(a.n_tiles, m_blocks), block(W * kWave);
  const size_t shm = (size_t)W * MT * kWave * sizeof(f32x4_t);
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_gemm<T, 1, EPI, KPW>), grid, block, shm, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<T, 2, EPI, KPW>), grid, block, shm, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<T, 3, EPI, KPW>), grid, block, shm, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<T, 4, EPI, KPW>), grid, block, shm, st, a); break;
  }
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_gemm_epi(const GemmArgs& a, int kpw, int MT, hipStream_t st) {
  switch (kpw) {
    case 1: return launch_gemm_kpw<T, EPI, 1>(a, MT, st);
    case 2: return launch_gemm_kpw<T, EPI, 2>(a, MT, st);
    case 4: return launch_gemm_kpw<T, EPI, 4>(a, MT, st);
    default: return launch_gemm_kpw<T, EPI, 8>(a, MT, st);
  }
}

template <typename T>
hipError_t launch_gemm(const GemmArgs& a, int epi, int kpw, hipStream_t st) {
  const int MT = a.M <= 16 ? 1 : a.M <= 32 ? 2 : a.M <= 48 ? 3 : 4;
  switch (epi) {
    case EPI_QKV: return launch_gemm_epi<T, EPI_QKV>(a, kpw, MT, st);
    case EPI_RESID: return launch_gemm_epi<T, EPI_RESID>(a, kpw, MT, st);
    case EPI_SWIGLU: return launch_gemm_epi<T, EPI_SWIGLU>(a, kpw, MT, st);
    default: return launch_gemm_epi<T, EPI_LOGITS>(a, kpw, MT, st);
  }
}
template hipError_t launch_gemm<bf16_t>(const GemmArgs&, int, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs&, int, int, hipStream_t);

hipError_t launch_argmax(const float* v1, const int32_t* i1, const float* v2, int n_groups, int ld, int M,
                         int32_t* tok, float* top1, float* top2, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax, dim3(M), dim3(kThreads), 0, st, v1, i1, v2, n_groups, ld, tok, top1, top2);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn(const AttnArgs& a, int n_chunk_slots, int head_dim, hipStream_t st) {
  dim3 grid(a.fold ? 1 : n_chunk_slots, a.n_kv, a.tasks.n);
  if (head_dim == 64) hipLaunchKernelGGL((k_attn<T, 64>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((k_attn<T, 32>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_attn<bf16_t>(const AttnArgs&, int, int, hipStream_t);
template hipError_t launch_attn<float>(const AttnArgs&, int, int, hipStream_t);

template <typename T>
hipError_t launch_attn_combine(const float* part, int max_chunks, int n_heads, int head_dim,
                               const int32_t* row_lim, int M, void* out, int out_ld, hipStream_t st) {
  const int blocks = (M * n_heads + 3) / 4;
  if (head_dim == 64)
    hipLaunchKernelGGL((k_attn_combine<T, 64>), dim3(blocks), dim3(kThreads), 0, st, part, max_chunks,
                       n_heads, row_lim, M, out, out_ld);
  else
    hipLaunchKernelGGL((k_attn_combine<T, 32>), dim3(blocks), dim3(kThreads), 0, st, part, max_chunks,
                       n_heads, row_lim, M, out, out_ld);
  return hipGetLastError();
}
template hipError_t launch_attn_combine<bf16_t>(const float*, int, int, int, const int32_t*, int, void*, int,
                                                hipStream_t);
template hipError_t launch_attn_combine<float>(const float*, int, int, int, const int32_t*, int, void*, int,
                                               hipStream_t);

hipError_t launch_accept(const int32_t* row_tok, const int32_t* am, const ReqArgs* ra, int n_req, int eos_id,
                         int32_t* out, int out_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_accept, dim3(n_req), dim3(64), 0, st, row_tok, am, ra, eos_id, out, out_stride);
  return hipGetLastError();
}

}  // namespace ssb
