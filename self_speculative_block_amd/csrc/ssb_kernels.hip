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
#include "ssb_device.h"

namespace ssb {

// ---------------------------------------------------------------------------
// Weight packing: W[N][K] row-major -> tiles [n_tile][k_step][lane][16 bytes],
// lane l of (tile t, step s) holding row 16t + l%16, K values
// s*kStepK + (kStepK/4)*(l/16) ... +kStepK/4.  One wave then reads 1 KiB of
// contiguous memory per step and feeds it straight to the matrix core.
// Row sources: mode 0 = rows of src0 (rows >= n0 are zero padding);
// mode 1 = concatenation src0 (n0 rows) | src1 (n1 rows) | src2 (rest);
// mode 2 = SwiGLU interleave: packed group j of 64 rows holds rows
// 32j..32j+31 of src0 (gate) then the same rows of src1 (up).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void k_pack(uint4* dst, int n_tiles, int K, int mode, const T* src0, const T* src1,
                       const T* src2, int n0, int n1) {
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
    const int row = tile * 16 + lane % 16;
    const int k = step * KS + PER * (lane / 16);
    const T* src = nullptr;
    int srow = row;
    if (mode == 0) {
      if (row < n0) src = src0;
    } else if (mode == 1) {
      if (row < n0) src = src0;
      else if (row < n0 + n1) { src = src1; srow = row - n0; }
      else { src = src2; srow = row - n0 - n1; }
    } else {
      const int j = row / 64, i = row % 64;
      src = i < 32 ? src0 : src1;
      srow = 32 * j + (i % 32);
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src) v = *reinterpret_cast<const uint4*>(src + (size_t)srow * K + k);
    dst[f] = v;
  }
}

// ---------------------------------------------------------------------------
// Row preparation + embedding gather.  Writes the per-row metadata of a
// forward (token, position, visibility limit, request) and the fp32 residual
// h = E[token] (or a prefix-embedding row), plus per-64-column sums of
// squares of h used by the next RMSNorm.
// ---------------------------------------------------------------------------


__device__ __forceinline__ void window_row(const PrepArgs& a, int m, int& tok, int& pos, int& lim,
                                           int& req) {
  if (a.mode == PREP_PREFILL) {
    tok = -1; pos = a.pos0 + m; lim = pos; req = 0;
  } else if (a.mode == PREP_TOKENS) {
    tok = a.tokens[m]; pos = a.pos0 + m; lim = pos; req = 0;
  } else {
    const int W = a.req.B + 1;
    const int r = m / W, j = m % W;
    req = r;
    const int p = a.req.p[r];
    if (a.mode == PREP_DRAFT) {
      // draft window: boundary x0 at p (causal), masks at p+1..p+B (see the window)
      tok = j == 0 ? a.req.x0[r] : a.mask_id;
      pos = p + j;
      lim = j == 0 ? p : p + a.req.B;
    } else {
      // verify window [a0, d1..dB] at p+1..p+B+1, causal; row j of the draft
      // predicted a0 (j = 0) or d_j
      pos = p + 1 + j;
      lim = pos;
      tok = a.am_prev[m];
      if (j >= 1) {
        int pl = -1;
        if (a.req.planted[r]) {
          pl = a.req.planted[r][j - 1];
        } else if (a.req.cont[r]) {
          const int idx = a.req.cont_c[r] + j;          // 0-based index of y_{c+1+j}
          const int as = a.req.astar[r];
          if (idx < a.req.cont_len[r]) {
            if (j <= as) pl = a.req.cont[r][idx];
            else if (j == as + 1) pl = (a.req.cont[r][idx] + 1) % (a.vocab - 1);
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
  const int col = g * kNormGroup + t;
  const T* src = tok >= 0 ? reinterpret_cast<const T*>(a.embed) + (size_t)tok * a.hidden
                          : reinterpret_cast<const T*>(a.prefix) + (size_t)pos * a.hidden;
  const float v = Ty<T>::to_f(src[col]);
  a.h[(size_t)m * a.hidden + col] = v;
  float s = v * v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
  if (t == 0) a.ssq[(size_t)g * a.ssq_ld + m] = s;
}

// ---------------------------------------------------------------------------
// Small-M / large-M GEMM with fused epilogues.
//   out[m][n] = sum_k X[m][k] * W[n][k]
// Grid: (n_groups, S, m_blocks).  A workgroup owns NT n-tiles (NG = 16*NT
// output columns) of one m-block (16*MT rows) and K chunks
// [split*cps, (split+1)*cps) of the fixed 128-wide chunks.  Each chunk is
// reduced from zero and added to the running sum in chunk order; with S > 1
// every split writes its sum and the last workgroup to arrive (atomic ticket)
// adds the S split sums in split order.  The decomposition (S) is a fixed
// property of each weight matrix for all decode forwards, so a row's value
// never depends on M.
// RMSNorm inputs are consumed as X = h * gain (rounded to T) and each output
// row is scaled by 1/rms(h) in the epilogue; rms comes from the per-64-column
// sum-of-squares partials of h, added in column order.
// ---------------------------------------------------------------------------


template <typename T, int MT, bool NORM>
__device__ __forceinline__ void stage_x(unsigned char* xs, const GemmArgs& a, int m_base, int kc) {
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int FPR = kChunkK / PER;                         // fragments per row
  constexpr int XSTRIDE = kChunkK * (int)sizeof(T) + 16;
  for (int f = threadIdx.x; f < MT * 16 * FPR; f += kThreads) {
    const int r = f / FPR, q = f % FPR;
    const int m = m_base + r;
    const int k = kc * kChunkK + q * PER;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < a.M) {
      if constexpr (NORM) {
        const float* hp = a.h + (size_t)m * a.hidden + k;
        const float* gp = a.gain + k;
        if constexpr (sizeof(T) == 2) {
          float4 h0 = *reinterpret_cast<const float4*>(hp);
          float4 h1 = *reinterpret_cast<const float4*>(hp + 4);
          float4 g0 = *reinterpret_cast<const float4*>(gp);
          float4 g1 = *reinterpret_cast<const float4*>(gp + 4);
          v.x = (uint32_t)f2bf(h0.x * g0.x) | ((uint32_t)f2bf(h0.y * g0.y) << 16);
          v.y = (uint32_t)f2bf(h0.z * g0.z) | ((uint32_t)f2bf(h0.w * g0.w) << 16);
          v.z = (uint32_t)f2bf(h1.x * g1.x) | ((uint32_t)f2bf(h1.y * g1.y) << 16);
          v.w = (uint32_t)f2bf(h1.z * g1.z) | ((uint32_t)f2bf(h1.w * g1.w) << 16);
        } else {
          float4 h0 = *reinterpret_cast<const float4*>(hp);
          float4 g0 = *reinterpret_cast<const float4*>(gp);
          v.x = __float_as_uint(h0.x * g0.x); v.y = __float_as_uint(h0.y * g0.y);
          v.z = __float_as_uint(h0.z * g0.z); v.w = __float_as_uint(h0.w * g0.w);
        }
      } else {
        v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.x) + (size_t)m * a.ldx + k);
      }
    }
    *reinterpret_cast<uint4*>(xs + r * XSTRIDE + q * 16) = v;
  }
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <typename T, int NT, int MT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs a) {
  constexpr int NG = NT * 16;
  constexpr int MB = MT * 16;
  constexpr int KS = Ty<T>::kStepK;
  constexpr int PER = Ty<T>::kPerFrag;
  constexpr int STEPS = kChunkK / KS;
  constexpr int XSTRIDE = kChunkK * (int)sizeof(T) + 16;
  constexpr bool NORM = (EPI != EPI_RESID);
  constexpr int WPN = 4 / NT;          // waves sharing one n-tile (split over m-tiles)
  __shared__ __align__(16) unsigned char xs[MB * XSTRIDE];
  __shared__ float ctile[MB][NG + 4];
  __shared__ float s_inv[MB];
  __shared__ int s_last;

  const int grp = blockIdx.x, split = blockIdx.y, mblk = blockIdx.z;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nchunks = a.K / kChunkK;
  const int cps = nchunks / a.S;
  const int c0 = split * cps, c1 = c0 + cps;
  const int ksteps = a.K / KS;
  const int m_base = mblk * MB;
  const int nt = wave % NT;
  const int mt0 = wave / NT;
  const int tile = grp * NT + nt;
  const uint4* wp = a.W + (size_t)tile * ksteps * kWave + lane;
  const int Ntot = a.n_groups * NG;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wnext[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) wnext[s] = wp[(size_t)(c0 * STEPS + s) * kWave];

  for (int c = c0; c < c1; ++c) {
    uint4 wcur[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) wcur[s] = wnext[s];
    if (c + 1 < c1) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) wnext[s] = wp[(size_t)((c + 1) * STEPS + s) * kWave];
    }
    stage_x<T, MT, NORM>(xs, a, m_base, c);
    __syncthreads();
    f32x4_t accc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) accc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt % WPN != mt0) continue;
        const uint4 b = *reinterpret_cast<const uint4*>(
            xs + (mt * 16 + lane % 16) * XSTRIDE + (s * KS + PER * (lane / 16)) * (int)sizeof(T));
        mma_step(accc[mt], wcur[s], b, T());
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt % WPN == mt0) acc[mt] += accc[mt];
    __syncthreads();
  }

  if (a.S > 1) {
    // publish this split's sum, then the last arriving workgroup adds all splits in order
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt % WPN != mt0) continue;
      const int m = m_base + mt * 16 + lane % 16;
      if (m < a.M) {
        float* dst = a.part + ((size_t)split * a.M + m) * Ntot + grp * NG + nt * 16 + 4 * (lane / 16);
        *reinterpret_cast<f32x4_t*>(dst) = acc[mt];
      }
    }
    __threadfence();
    __syncthreads();
    const int ctr = grp * gridDim.z + mblk;
    if (threadIdx.x == 0) s_last = (atomicAdd(&a.counters[ctr], 1) == a.S - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt % WPN != mt0) continue;
      acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int m = m_base + mt * 16 + lane % 16;
      if (m < a.M) {
        for (int s = 0; s < a.S; ++s) {
          const float* src = a.part + ((size_t)s * a.M + m) * Ntot + grp * NG + nt * 16 + 4 * (lane / 16);
          acc[mt] += *reinterpret_cast<const f32x4_t*>(src);
        }
      }
    }
    if (threadIdx.x == 0) a.counters[ctr] = 0;
  }

  // full tile -> LDS
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt % WPN != mt0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) ctile[mt * 16 + lane % 16][nt * 16 + 4 * (lane / 16) + i] = acc[mt][i];
  }
  if constexpr (NORM) {
    for (int r = threadIdx.x; r < MB; r += kThreads) {
      const int m = m_base + r;
      float s = 0.f;
      if (m < a.M)
        for (int g = 0; g < a.n_ssq; ++g) s += a.ssq[(size_t)g * a.ssq_ld + m];
      s_inv[r] = 1.0f / sqrtf(s / (float)a.hidden + a.eps);
    }
  }
  __syncthreads();

  if constexpr (EPI == EPI_QKV) {
    const int hd = a.head_dim, half = hd / 2;
    const int kind = grp < a.n_heads ? 0 : (grp < a.n_heads + a.n_kv ? 1 : 2);   // q, k, v
    const int head = kind == 0 ? grp : (kind == 1 ? grp - a.n_heads : grp - a.n_heads - a.n_kv);
    for (int e = threadIdx.x; e < MB * half; e += kThreads) {
      const int r = e / half, i = e % half;
      const int m = m_base + r;
      if (m >= a.M) continue;
      const float inv = s_inv[r];
      float x1 = ctile[r][i] * inv, x2 = ctile[r][i + half] * inv;
      const int pos = a.row_pos[m];
      if (kind != 2) {
        const float2 cs = a.rope[(size_t)pos * half + i];
        const float o1 = x1 * cs.x - x2 * cs.y;
        const float o2 = x2 * cs.x + x1 * cs.y;
        x1 = o1; x2 = o2;
      }
      T* dst;
      if (kind == 0) {
        dst = reinterpret_cast<T*>(a.y) + (size_t)m * a.ldy + head * hd;
      } else {
        const int32_t* pt = a.pt[a.row_req[m]];
        const int page = pt[pos / kPage], slot = pos % kPage;
        const size_t base = (((size_t)a.layer * a.n_pages + page) * 2 + (kind - 1)) * a.n_kv + head;
        dst = reinterpret_cast<T*>(a.kv_pool) + (base * kPage + slot) * hd;
      }
      dst[i] = Ty<T>::from_f(x1);
      dst[i + half] = Ty<T>::from_f(x2);
    }
  } else if constexpr (EPI == EPI_RESID) {
    for (int e = threadIdx.x; e < MB * NG; e += kThreads) {
      const int r = e / NG, n = e % NG;
      const int m = m_base + r;
      if (m >= a.M) continue;
      float* hp = a.h_out + (size_t)m * a.hidden + grp * NG + n;
      const float v = *hp + ctile[r][n];
      *hp = v;
      ctile[r][n] = v;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < MB; r += kThreads) {
      const int m = m_base + r;
      if (m >= a.M) continue;
      float s = 0.f;
      for (int n = 0; n < NG; ++n) s += ctile[r][n] * ctile[r][n];
      a.ssq_out[(size_t)grp * a.ssq_ld + m] = s;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HG = NG / 2;
    for (int e = threadIdx.x; e < MB * HG; e += kThreads) {
      const int r = e / HG, i = e % HG;
      const int m = m_base + r;
      if (m >= a.M) continue;
      const float g = ctile[r][i] * s_inv[r];
      const float u = ctile[r][HG + i] * s_inv[r];
      reinterpret_cast<T*>(a.y)[(size_t)m * a.ldy + grp * HG + i] = Ty<T>::from_f(silu_f(g) * u);
    }
  } else {  // EPI_LOGITS
    for (int e = threadIdx.x; e < MB * NG; e += kThreads) {
      const int r = e / NG, n = e % NG;
      const int m = m_base + r;
      const float z = ctile[r][n] * s_inv[r];
      ctile[r][n] = z;
      const int col = grp * NG + n;
      if (a.logits && m < a.M && col < a.vocab) a.logits[(size_t)m * a.vocab + col] = z;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < MB; r += kThreads) {
      const int m = m_base + r;
      if (m >= a.M) continue;
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7fffffff;
      bool nan = false;
      for (int n = 0; n < NG; ++n) {
        const int col = grp * NG + n;
        if (col >= a.vocab || col == a.mask_id) continue;
        const float z = ctile[r][n];
        if (z != z) { nan = true; continue; }
        if (z > v1) { v2 = v1; v1 = z; i1 = col; }
        else if (z > v2) { v2 = z; }
      }
      if (nan) { v1 = NAN; v2 = NAN; i1 = -1; }
      a.am_v1[(size_t)grp * a.am_ld + m] = v1;
      a.am_i1[(size_t)grp * a.am_ld + m] = i1;
      a.am_v2[(size_t)grp * a.am_ld + m] = v2;
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
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  for (int g = threadIdx.x; g < n_groups; g += kThreads)
    t = merge_top2(t, Top2{v1[(size_t)g * ld + m], i1[(size_t)g * ld + m], v2[(size_t)g * ld + m]});
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
// in the lanes that feed P^T to the V^T P^T product without shuffles.
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
  constexpr int KSTR = HD * (int)sizeof(T) + 16;
  constexpr int MT = kTaskRows / 16;
  constexpr int REC = HD + 4;
  __shared__ __align__(16) unsigned char ks[kKeyChunk * KSTR];
  __shared__ __align__(16) unsigned char vs[kKeyChunk * KSTR];
  __shared__ int s_lim[kTaskRows];
  __shared__ int s_maxlim;

  const AttnTask task = a.tasks.t[blockIdx.z];
  const int g = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n_rep = a.n_heads / a.n_kv;
  const int32_t* pt = a.pt[task.req];

  if (threadIdx.x < kTaskRows)
    s_lim[threadIdx.x] = threadIdx.x < task.nrows ? a.row_lim[task.row0 + threadIdx.x] : -1;
  __syncthreads();
  if (threadIdx.x == 0) {
    int mx = -1;
    for (int r = 0; r < task.nrows; ++r) mx = max(mx, s_lim[r]);
    s_maxlim = mx;
  }
  __syncthreads();
  const int maxlim = s_maxlim;
  int cbeg, cend;
  if (a.fold) { cbeg = 0; cend = maxlim / kKeyChunk + 1; }
  else {
    cbeg = blockIdx.x; cend = cbeg + 1;
    if (cbeg * kKeyChunk > maxlim) return;
  }

  // units: (head within group, row tile) handled by this wave
  const int n_units = n_rep * MT;
  constexpr int MAXU = 3;                  // ceil(4 heads * 3 tiles / 4 waves)
  float run_m[MAXU], run_l[MAXU];
  f32x4_t run_o[MAXU][DT];
#pragma unroll
  for (int u = 0; u < MAXU; ++u) {
    run_m[u] = -INFINITY; run_l[u] = 0.f;
#pragma unroll
    for (int d = 0; d < DT; ++d) run_o[u][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int c = cbeg; c < cend; ++c) {
    // stage K and V of keys [c*64, c*64+64) that any row of the task may see
    constexpr int FPK = HD / PER;          // 16-byte fragments per key row
    for (int f = threadIdx.x; f < 2 * kKeyChunk * FPK; f += kThreads) {
      const int kv = f / (kKeyChunk * FPK);
      const int rem = f % (kKeyChunk * FPK);
      const int kk = rem / FPK, q = rem % FPK;
      const int key = c * kKeyChunk + kk;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key <= maxlim) {
        const int page = pt[key / kPage], slot = key % kPage;
        const size_t base = (((size_t)a.layer * a.n_pages + page) * 2 + kv) * a.n_kv + g;
        v = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.kv_pool) +
                                            (base * kPage + slot) * HD + q * PER);
      }
      *reinterpret_cast<uint4*>((kv ? vs : ks) + kk * KSTR + q * 16) = v;
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
      // Q^T fragments (B operand): row_local's query, head dims of this lane
      uint4 qf[QKS];
#pragma unroll
      for (int st = 0; st < QKS; ++st) {
        qf[st] = make_uint4(0, 0, 0, 0);
        if (row_local < task.nrows)
          qf[st] = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const T*>(a.q) + (size_t)(task.row0 + row_local) * a.q_ld + head * HD +
              st * KS + PER * (lane / 16));
      }
      // S^T tiles: element i of tile kt = score of key kt*16 + 4*(lane/16) + i for row_local
      f32x4_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QKS; ++st) {
          const uint4 kf = *reinterpret_cast<const uint4*>(
              ks + (kt * 16 + lane % 16) * KSTR + (st * KS + PER * (lane / 16)) * (int)sizeof(T));
          mma_step(s[kt], kf, qf[st], T());
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
#pragma unroll
        for (int st = 0; st < PVS; ++st) {
          uint4 pf, vf;
          if constexpr (sizeof(T) == 2) {
            // keys 32st + 4(l/16) + {0..3} from tile 2st, then +16 from tile 2st+1
            const f32x4_t p0 = s[2 * st], p1 = s[2 * st + 1];
            pf.x = (uint32_t)f2bf(p0[0]) | ((uint32_t)f2bf(p0[1]) << 16);
            pf.y = (uint32_t)f2bf(p0[2]) | ((uint32_t)f2bf(p0[3]) << 16);
            pf.z = (uint32_t)f2bf(p1[0]) | ((uint32_t)f2bf(p1[1]) << 16);
            pf.w = (uint32_t)f2bf(p1[2]) | ((uint32_t)f2bf(p1[3]) << 16);
            const int d = dt * 16 + lane % 16;
            uint16_t vv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int key = 32 * st + (j < 4 ? 4 * (lane / 16) + j : 16 + 4 * (lane / 16) + j - 4);
              vv[j] = *reinterpret_cast<const uint16_t*>(vs + key * KSTR + d * 2);
            }
            vf.x = vv[0] | ((uint32_t)vv[1] << 16); vf.y = vv[2] | ((uint32_t)vv[3] << 16);
            vf.z = vv[4] | ((uint32_t)vv[5] << 16); vf.w = vv[6] | ((uint32_t)vv[7] << 16);
          } else {
            const f32x4_t p0 = s[st];
            pf = make_uint4(__float_as_uint(p0[0]), __float_as_uint(p0[1]), __float_as_uint(p0[2]),
                            __float_as_uint(p0[3]));
            const int d = dt * 16 + lane % 16;
            uint32_t vv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = 16 * st + 4 * (lane / 16) + j;
              vv[j] = *reinterpret_cast<const uint32_t*>(vs + key * KSTR + d * 4);
            }
            vf = make_uint4(vv[0], vv[1], vv[2], vv[3]);
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
// One wave per (row, head); lane d holds output dimension d.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_combine(const float* part, int max_chunks, int n_heads,
                                                          const int32_t* row_lim, int M, void* out,
                                                          int out_ld) {
  constexpr int REC = HD + 4;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= M * n_heads) return;
  const int row = idx / n_heads, head = idx % n_heads;
  const int nch = row_lim[row] / kKeyChunk + 1;
  const float* rec = part + ((size_t)row * n_heads + head) * max_chunks * REC;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float mc = rec[c * REC + HD], lc = rec[c * REC + HD + 1];
    const float oc = lane < HD ? rec[c * REC + lane] : 0.f;
    float mn, al, be;
    fold_coef(m, mc, mn, al, be);
    l = fold_val(l, al, lc, be);
    o = fold_val(o, al, oc, be);
    m = mn;
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
__global__ __launch_bounds__(64) void k_accept(const int32_t* row_tok, const int32_t* am, ReqArgs ra,
                                               int eos_id, int32_t* out, int out_stride) {
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
                       const void* s2, int n0, int n1, hipStream_t st) {
  hipLaunchKernelGGL(k_pack<T>, dim3(1024), dim3(256), 0, st, dst, n_tiles, K, mode,
                     (const T*)s0, (const T*)s1, (const T*)s2, n0, n1);
  return hipGetLastError();
}
template hipError_t launch_pack<bf16_t>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                        int, hipStream_t);
template hipError_t launch_pack<float>(uint4*, int, int, int, const void*, const void*, const void*, int,
                                       int, hipStream_t);

template <typename T>
hipError_t launch_prep(const PrepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_prep_embed<T>, dim3(a.M, a.hidden / kNormGroup), dim3(64), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_prep<bf16_t>(const PrepArgs&, hipStream_t);
template hipError_t launch_prep<float>(const PrepArgs&, hipStream_t);

template <typename T, int NT, int EPI>
static hipError_t launch_gemm_nt(const GemmArgs& a, int m_blocks, int MT, hipStream_t st) {
  dim3 grid(a.n_groups, a.S, m_blocks);
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_gemm<T, NT, 1, EPI>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemm<T, NT, 2, EPI>), grid, dim3(kThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemm<T, NT, 3, EPI>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemm<T, NT, 4, EPI>), grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm(const GemmArgs& a, int epi, int nt, hipStream_t st) {
  const int MT = a.M <= 16 ? 1 : a.M <= 32 ? 2 : a.M <= 48 ? 3 : 4;
  const int m_blocks = (a.M + 16 * MT - 1) / (16 * MT);
  if (epi == EPI_QKV) {
    return nt == 2 ? launch_gemm_nt<T, 2, EPI_QKV>(a, m_blocks, MT, st)
                   : launch_gemm_nt<T, 4, EPI_QKV>(a, m_blocks, MT, st);
  }
  if (epi == EPI_RESID) return launch_gemm_nt<T, 4, EPI_RESID>(a, m_blocks, MT, st);
  if (epi == EPI_SWIGLU) return launch_gemm_nt<T, 4, EPI_SWIGLU>(a, m_blocks, MT, st);
  return launch_gemm_nt<T, 4, EPI_LOGITS>(a, m_blocks, MT, st);
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

hipError_t launch_accept(const int32_t* row_tok, const int32_t* am, const ReqArgs& ra, int eos_id,
                         int32_t* out, int out_stride, hipStream_t st) {
  hipLaunchKernelGGL(k_accept, dim3(ra.n), dim3(64), 0, st, row_tok, am, ra, eos_id, out, out_stride);
  return hipGetLastError();
}

}  // namespace ssb
