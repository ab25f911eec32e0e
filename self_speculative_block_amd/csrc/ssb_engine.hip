// Host engine and C ABI of the self-speculative round (see include/ssb.h).
//
// The engine owns: the packed weights, a fixed workspace (allocated once at
// init), the KV page allocator and the orchestration of forwards.  Every
// forward is a fixed sequence of kernel launches on the caller's stream:
//   prep+embed, then per layer [QKV+RoPE+KV write, attention (+combine),
//   O + residual, gate|up + SwiGLU, down + residual], then LM head + argmax.
// A round is draft forward, verify forward, accept, then one device->host
// copy of the committed tokens (GravityOCR review, section 3.2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>
#include <new>
#include <string>
#include <vector>

#include "../../include/ssb.h"
#include "ssb_device.h"
#include "ssb_host.h"


using namespace ssb;

namespace {

thread_local std::string g_err;

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(SSB_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <typename F>
int guard(F&& f) {
  const int rc = run_guarded(f, &g_err);
  if (rc != SSB_OK) ssb::g_prof_ev[0] = ssb::g_prof_ev[1] = nullptr;   // a launch that failed inside the timing hook
  return rc;
}

constexpr int kDDRec = 4 + 4 * SSB_MAX_BLOCK;      // direct-diffusion step record per request

}  // namespace

// A pool: the caller's KV buffer and its free page ids.
struct ssb_pool : PageStack {
  ssb_model* m;
  char* base;
};

// A sequence: its pages (logical page -> pool page), its committed state, and its page table on
// the device with a pinned host mirror (max_pages entries each).
struct ssb_kv : PageList, SeqState {
  ssb_pool* pool;
  int32_t* pt_dev;
  int32_t* pt_host;
};

struct GemmShape {
  const uint4* W;
  int K, n_tiles;        // reduction length, 16-column tiles
  int NT, KSL, S;        // tiles per workgroup, K slices per tile, K ranges
};

// Device buffers a forward pass and its accept step read and write, sized for the model's largest
// forward at init; ssb_round_noalloc lays out the same buffers for one window in the file-scope
// scratch array instead, for the length of the call.
struct Workspace {
  float* h;
  void* xg;
  float* ssq;
  void* q;
  void* attn;
  void* act;
  int32_t *row_tok, *row_pos, *row_lim, *row_req, *row_slot;
  float2* row_cs;
  float* part;        // K-split partial sums [S][max_rows][hidden]
  int32_t* fwd_pt;    // page ids of the current forward's requests [kMaxReq][pt_ld]
  int pt_ld;
  int32_t* am_tok;
  float *am_top1, *am_top2;
  float *amv1, *amv2;
  int32_t* ami1;
  float* ams;         // per-group softmax sums of the LM head (confidence, sampling)
  float* am_z;        // per row: sum of exp((z - max) / T) over the vocabulary without [M]
  float *slog_d, *slog_v;   // stochastic rounds: draft / verify logits [max_decode_rows][vocab]
  float *smax_d, *sz_d, *smax_v, *sz_v;   // their row max and exp-sum [max_rows]
  int32_t* dd_win;    // block tokens of the direct-diffusion request [kMaxReq][SSB_MAX_BLOCK + 1]
  int32_t* dd_rec;    // step records [kMaxReq][kDDRec]
  float* apart;       // attention chunk records [max_decode_rows][n_heads][max_chunks][hd + 4]
  int max_chunks;
  int max_decode_rows;
  int32_t* accept_dev;
  int32_t* tok_dev;
  ReqArgs* req_dev;   // device request state read by every kernel of a forward
};

struct ssb_model : Workspace {
  ssb_config c;
  int device;
  int elem;
  // packed weights
  void* wmem;
  size_t wmem_bytes = 0, ws_bytes = 0;
  const void* embed;
  const float* final_norm;
  std::vector<const float*> attn_norm, mlp_norm;
  std::vector<GemmShape> qkv, o, gu, d;
  GemmShape lm;
  float2* rope;
  // workspace allocation (the Workspace pointers point into it)
  void* ws;
  int max_batch;      // requests per batched call
  bool sampling;      // stochastic-round workspace allocated
  bool no_graph = false;       // launches run eagerly (ssb_round_noalloc: instantiating a graph allocates)
  bool debug_poison = false;   // NaN-poison KV slots no correct read reaches (rounds run eagerly)
  // fused layer tail (O, gate|up, down in one launch) for decode forwards of <= 48 rows
  bool tail_ok = false;        // the model's shapes and the device allow it
  bool no_fused = false;       // debug: always run the three GEMM launches
  unsigned long long* tail_sync = nullptr;   // barrier counters and generation [kTailSyncWords]
  int* tail_err = nullptr;     // set by a layer-tail barrier that timed out
  ReqArgs* req_pin;   // pinned staging of the request state
  hipStream_t cap;    // private stream used only to capture graphs
  std::map<std::tuple<int, void*, int, int, uint32_t, int>, hipGraphExec_t> graphs;   // (kind, pool, R, B, T bits, slots)
  // kernel timing hook
  int prof_kind = -1;
  bool prof_graph = false;            // time launches of prof_kind inside graph replays (device stamps)
  bool capturing = false;             // a launch graph is being captured on m->cap
  // kinds of the launches of each graph captured for timing, in launch order (one stamp slot each)
  std::map<hipGraphExec_t, std::vector<int>> graph_prof_kinds;
  ProfStamp* prof_stamps = nullptr;   // device slots of graph-replayed launches [prof_slots]
  int prof_slots = 0;
  int prof_stamp_used = 0;            // slots the last replayed graph wrote
  std::vector<int> prof_cap_kinds;    // kinds of the slots of the graph being captured / replayed
  double wallclock_mhz = 100.0;       // device real-time counter
  std::vector<hipEvent_t> prof_ev;    // pairs (start, end)
  int prof_used = 0;                  // pairs recorded since the last collect
  double prof_us = 0;
  long long prof_launches = 0;
  // pinned host staging
  int32_t* pin_i32;   // [max_rows + kMaxReq*kOutStride]
  float* pin_f32;     // [2*max_rows]
};

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Kinds of launches that are never timed themselves but stamp their end in a timing graph (the
// interval of the launch after them starts there).
constexpr int kKindPrep = 100, kKindAccept = 101;

// Kernel timing hook around each launch of the selected kind.  Eager launches carry a start /
// stop event pair on the dispatch itself (hipExtLaunchKernel).  In a graph captured for timing
// every launch gets a device stamp slot instead (latest workgroup end on the real-time counter;
// HIP cannot time events recorded by graph nodes), and a launch of the selected kind is timed
// from the end of the launch before it to its own end: back-to-back graph launches start when
// the previous one completes, so this is the interval a kernel trace reports for the dispatch.
ProfStamp* prof_begin(ssb_model* m, int kind, hipStream_t) {
  if (m->capturing) {
    if (!m->prof_graph) return nullptr;
    if (m->prof_stamp_used >= m->prof_slots) fail(SSB_EINVAL, "kernel timing: too many launches per graph");
    m->prof_cap_kinds.push_back(kind);
    return m->prof_stamps + m->prof_stamp_used;
  }
  if (m->prof_kind != kind) return nullptr;
  if (m->prof_used * 2 + 2 > (int)m->prof_ev.size()) fail(SSB_EINVAL, "kernel timing: too many launches per call");
  g_prof_ev[0] = m->prof_ev[2 * m->prof_used];
  g_prof_ev[1] = m->prof_ev[2 * m->prof_used + 1];
  return nullptr;
}
void prof_end(ssb_model* m, int kind, hipStream_t) {
  if (m->capturing) {
    if (m->prof_graph) ++m->prof_stamp_used;
    return;
  }
  if (m->prof_kind != kind) return;
  g_prof_ev[0] = g_prof_ev[1] = nullptr;
  ++m->prof_used;
}
// Rounds replay graphs unless a kind is timed eagerly.
bool prof_eager(const ssb_model* m) { return m->prof_kind >= 0 && !m->prof_graph; }
// Called after the stream has been synchronized.
void prof_collect(ssb_model* m) {
  for (int i = 0; i < m->prof_used; ++i) {
    float ms = 0.f;
    hip_check(hipEventElapsedTime(&ms, m->prof_ev[2 * i], m->prof_ev[2 * i + 1]), "profile elapsed");
    m->prof_us += ms * 1000.0;
  }
  m->prof_launches += m->prof_used;
  m->prof_used = 0;
  if (m->prof_stamp_used > 0) {
    const int n = m->prof_stamp_used;
    std::vector<ProfStamp> st(n);
    hip_check(hipMemcpy(st.data(), m->prof_stamps, n * sizeof(ProfStamp), hipMemcpyDeviceToHost), "read stamps");
    // latest workgroup end of a slot; end words older than the launch's start belong to earlier
    // replays of the slot
    auto end_of = [](const ProfStamp& x) {
      unsigned long long t1 = 0;
      for (int w = 1; w <= kStampWgs; ++w)
        if (x.t[w] >= x.t[0] && x.t[w] > t1) t1 = x.t[w];
      return t1;
    };
    for (int i = 1; i < n && i < (int)m->prof_cap_kinds.size(); ++i) {
      if (m->prof_cap_kinds[i] != m->prof_kind) continue;
      const unsigned long long e0 = end_of(st[i - 1]), e1 = end_of(st[i]);
      if (e0 == 0 || e1 <= e0) continue;
      m->prof_us += (double)(e1 - e0) / m->wallclock_mhz;
      ++m->prof_launches;
    }
    m->prof_stamp_used = 0;
  }
}

// Workgroup shape of a GEMM: NT 16-column tiles per workgroup, KSL K slices
// per tile (8 waves in all), and, for a residual GEMM whose K is too long for
// one workgroup (EPI_PARTIAL requested), S K ranges over the grid's y axis
// (its epilogue then runs in k_resid_reduce).  Each wave chains 4..16 K steps
// (bf16) or 1..4 (f32).  The shape depends on the GEMM's dimensions only,
// never on the row count.
// Decode forwards of many rows (batched rounds) run a layer GEMM in the large-tile kernel's
// exact form from these row counts on (measured crossovers against k_gemm's looped form at
// 132 / 264 / 528 / 1040 rows: QKV 17 vs 26 us at 528 rows, O and down 15 vs 23 and 38 vs 60 us
// at 1040, gate|up 75 vs 79 us at 1040 but 49 vs 43 at 528).
constexpr int kExactRowsQkv = 384, kExactRowsO = 768, kExactRowsGateUp = 1024, kExactRowsDown = 768;
constexpr int kExactRowsLm = 256;   // LM head (records only; softmax-sum launches stay on k_gemm)

GemmShape plan_gemm(int K, int n_tiles, int elem, int epi) {
  const int KS = elem == 2 ? 32 : 16, ksteps = K / KS;
  const int kmin = elem == 2 ? 4 : 1, kmax = elem == 2 ? 16 : 4;
  GemmShape g{};
  g.K = K;
  g.NT = epi == EPI_SWIGLU ? 2 : epi == EPI_LOGITS ? 4 : 1;
  g.KSL = epi == EPI_SWIGLU ? 4 : epi == EPI_LOGITS ? 2 : 8;
  g.S = 1;
  g.n_tiles = (n_tiles + g.NT - 1) / g.NT * g.NT;
  while (g.KSL > 1 && ksteps / (g.S * g.KSL) < kmin) g.KSL /= 2;
  while (ksteps / (g.S * g.KSL) > kmax) {
    if (g.NT * g.KSL < 8) g.KSL *= 2;
    else if (g.NT > 1 && n_tiles % (g.NT / 2) == 0) { g.NT /= 2; g.KSL *= 2; g.n_tiles = (n_tiles + g.NT - 1) / g.NT * g.NT; }
    else if (epi == EPI_PARTIAL && g.S < 8) g.S *= 2;   // split K over workgroups, reduced afterwards
    else fail(SSB_EINVAL, "reduction length too large for the GEMM kernel");
  }
  const int kpw = ksteps / (g.S * g.KSL);
  if (kpw < kmin || g.S * g.KSL * kpw != ksteps) fail(SSB_EINVAL, "reduction length too small for the GEMM kernel");
  return g;
}

template <typename T>
void pack_all(ssb_model* m, const ssb_weights* w, hipStream_t st) {
  const ssb_config& c = m->c;
  const int H = c.hidden, F = c.ffn, qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  // bf16 weights go into the packed copy as fp16: one flag word reports a value beyond fp16's range
  int* range_err = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&range_err), sizeof(int)) != hipSuccess)
    fail(SSB_ENOMEM, "allocation of the packing flag failed");
  std::unique_ptr<int, void (*)(int*)> hold(range_err, [](int* p) { (void)hipFree(p); });
  hip_check(hipMemsetAsync(range_err, 0, sizeof(int), st), "clear packing flag");
  for (int l = 0; l < c.n_layers; ++l) {
    hip_check(launch_pack<T>(const_cast<uint4*>(m->qkv[l].W), (qd + 2 * kvd) / 16, H, 1, w->wq[l], w->wk[l],
                             w->wv[l], qd, kvd, c.head_dim, range_err, st), "pack qkv");
    hip_check(launch_pack<T>(const_cast<uint4*>(m->o[l].W), H / 16, qd, 0, w->wo[l], nullptr, nullptr, H, 0, 0,
                             range_err, st), "pack o");
    hip_check(launch_pack<T>(const_cast<uint4*>(m->gu[l].W), 2 * F / 16, H, 2, w->wg[l], w->wu[l], nullptr, 0, 0, 0,
                             range_err, st), "pack gate/up");
    hip_check(launch_pack<T>(const_cast<uint4*>(m->d[l].W), H / 16, F, 0, w->wd[l], nullptr, nullptr, H, 0, 0,
                             range_err, st), "pack down");
  }
  hip_check(launch_pack<T>(const_cast<uint4*>(m->lm.W), m->lm.n_tiles, H, 0, w->lm_head, nullptr, nullptr,
                           c.vocab, 0, 0, range_err, st), "pack lm_head");
  int bad = 0;
  hip_check(hipMemcpyAsync(&bad, range_err, sizeof(int), hipMemcpyDeviceToHost, st), "read packing flag");
  hip_check(hipStreamSynchronize(st), "packing");
  if (bad) fail(SSB_EINVAL, "a bf16 weight exceeds the fp16 range (|w| > 65504) of the packed copy");
}

void scratch_setup(int dev);   // the scratch array's device address (defined with the array)

void init_model(const ssb_config* cfg, const ssb_weights* w, hipStream_t st, ssb_model** out) {
  check_config(cfg);
  if (!w || !out) fail(SSB_EINVAL, "null weights or output pointer");
  const ssb_config& c = *cfg;
  auto* m = new ssb_model();
  std::unique_ptr<ssb_model> hold(m);
  m->c = c;
  hip_check(hipGetDevice(&m->device), "hipGetDevice");
  m->elem = c.dtype == SSB_BF16 ? 2 : 4;
  const int H = c.hidden, F = c.ffn, V = c.vocab, L = c.n_layers;
  const int qd = c.n_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const size_t E = m->elem;

  // ---- packed weights ----
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t o_embed = take((size_t)V * H * E);
  const size_t o_fnorm = take((size_t)H * 4);
  std::vector<size_t> o_an(L), o_mn(L), o_qkv(L), o_o(L), o_gu(L), o_d(L);
  for (int l = 0; l < L; ++l) {
    o_an[l] = take((size_t)H * 4);
    o_mn[l] = take((size_t)H * 4);
    o_qkv[l] = take((size_t)(qd + 2 * kvd) * H * E);
    o_o[l] = take((size_t)H * qd * E);
    o_gu[l] = take((size_t)2 * F * H * E);
    o_d[l] = take((size_t)H * F * E);
  }
  const GemmShape p_qkv = plan_gemm(H, (qd + 2 * kvd) / 16, (int)E, EPI_QKV);
  const GemmShape p_o = plan_gemm(qd, H / 16, (int)E, EPI_RESID);
  const GemmShape p_gu = plan_gemm(H, 2 * F / 16, (int)E, EPI_SWIGLU);
  const GemmShape p_d = plan_gemm(F, H / 16, (int)E, EPI_PARTIAL);
  const GemmShape p_lm = plan_gemm(H, (V + 15) / 16, (int)E, EPI_LOGITS);
  {
    auto fits = [&](const GemmShape& g, int epi) {
      if (gemm_max_mt((int)E, g.K, g.S, g.NT, g.KSL, H / 16, epi) < 1)
        fail(SSB_EINVAL, "GEMM slab does not fit in LDS for this configuration");
    };
    fits(p_qkv, EPI_QKV); fits(p_o, EPI_RESID); fits(p_gu, EPI_SWIGLU);
    fits(p_d, p_d.S > 1 ? EPI_PARTIAL : EPI_RESID); fits(p_lm, EPI_LOGITS);
  }
  const int lm_tiles = p_lm.n_tiles;
  const size_t o_lm = take((size_t)lm_tiles * 16 * H * E);
  const size_t o_rope = take((size_t)c.max_positions * (c.head_dim / 2) * sizeof(float2));
  if (hipMalloc(&m->wmem, off) != hipSuccess) fail(SSB_ENOMEM, "hipMalloc of packed weights failed");
  m->wmem_bytes = off;
  char* wb = static_cast<char*>(m->wmem);
  m->embed = wb + o_embed;
  m->final_norm = reinterpret_cast<const float*>(wb + o_fnorm);
  const int hd = c.head_dim;
  for (int l = 0; l < L; ++l) {
    m->attn_norm.push_back(reinterpret_cast<const float*>(wb + o_an[l]));
    m->mlp_norm.push_back(reinterpret_cast<const float*>(wb + o_mn[l]));
    m->qkv.push_back(p_qkv); m->qkv.back().W = reinterpret_cast<const uint4*>(wb + o_qkv[l]);
    m->o.push_back(p_o); m->o.back().W = reinterpret_cast<const uint4*>(wb + o_o[l]);
    m->gu.push_back(p_gu); m->gu.back().W = reinterpret_cast<const uint4*>(wb + o_gu[l]);
    m->d.push_back(p_d); m->d.back().W = reinterpret_cast<const uint4*>(wb + o_d[l]);
  }
  m->lm = p_lm;
  m->lm.W = reinterpret_cast<const uint4*>(wb + o_lm);
  m->rope = reinterpret_cast<float2*>(wb + o_rope);

  hip_check(hipMemcpyAsync(wb + o_embed, w->embed, (size_t)V * H * E, hipMemcpyDeviceToDevice, st), "copy embed");
  hip_check(hipMemcpyAsync(wb + o_fnorm, w->final_norm, (size_t)H * 4, hipMemcpyDeviceToDevice, st), "copy norm");
  for (int l = 0; l < L; ++l) {
    hip_check(hipMemcpyAsync(wb + o_an[l], w->attn_norm[l], (size_t)H * 4, hipMemcpyDeviceToDevice, st), "copy");
    hip_check(hipMemcpyAsync(wb + o_mn[l], w->mlp_norm[l], (size_t)H * 4, hipMemcpyDeviceToDevice, st), "copy");
  }
  if (c.dtype == SSB_BF16) pack_all<bf16_t>(m, w, st);
  else pack_all<float>(m, w, st);

  // RoPE table: angle = pos * theta^(-2i/hd), computed in double
  {
    const int half = hd / 2;
    std::vector<float2> tab((size_t)c.max_positions * half);
    for (int p = 0; p < c.max_positions; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * i / hd);
        tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    hip_check(hipMemcpyAsync(m->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, st),
              "copy rope");
    hip_check(hipStreamSynchronize(st), "init sync");
  }

  // ---- workspace ----
  const int MR = c.max_rows;
  m->max_batch = c.max_batch ? c.max_batch : SSB_MAX_BATCH;
  m->sampling = (c.features & SSB_FEAT_SAMPLE) != 0;
  m->max_decode_rows = std::min(MR, m->max_batch * (std::max(c.block_B, 1) + 1));
  m->max_chunks = (c.max_positions + kKeyChunk - 1) / kKeyChunk;
  off = 0;
  const size_t w_h = take((size_t)MR * H * 4);
  // activations that tall forwards keep fragment-major (whole 16-row tiles): rows rounded up to 16
  const int MR16 = (MR + 15) / 16 * 16;
  const size_t w_xg = take((size_t)MR16 * H * E);
  const size_t w_ssq = take((size_t)(H / 16) * MR * 4);
  const size_t w_q = take((size_t)MR * qd * E);
  const size_t w_attn = take((size_t)MR16 * qd * E);
  const size_t w_act = take((size_t)MR16 * F * E);
  const size_t w_meta = take((size_t)5 * MR * 4);
  const size_t w_cs = take((size_t)MR * (hd / 2) * sizeof(float2));
  m->pt_ld = m->max_chunks * (kKeyChunk / kPage);
  const size_t w_fpt = take((size_t)kMaxReq * m->pt_ld * 4);
  const size_t w_part = take((size_t)p_d.S * MR * H * 4);
  const size_t w_am = take((size_t)MR * 12);
  const size_t w_amp = take((size_t)(lm_tiles / p_lm.NT) * MR * 12);
  const size_t w_ams = take((size_t)(lm_tiles / p_lm.NT) * MR * 4);
  const size_t w_conf = take((size_t)MR * 4);
  const size_t w_slog = take(m->sampling ? (size_t)2 * m->max_decode_rows * V * 4 : 0);
  const size_t w_sst = take((size_t)4 * MR * 4);
  const size_t w_ddw = take((size_t)kMaxReq * (SSB_MAX_BLOCK + 1) * 4);
  const size_t w_ddr = take((size_t)kMaxReq * kDDRec * 4);
  const size_t w_apart = take((size_t)m->max_decode_rows * c.n_heads * m->max_chunks * (hd + 4) * 4);
  const size_t w_acc = take((size_t)kMaxReq * kOutStride * 4);
  const size_t w_tok = take((size_t)MR * 4);
  const size_t w_req = take(sizeof(ReqArgs));
  const size_t w_tail = take((size_t)kTailSyncWords * 8 + 256);
  if (hipMalloc(&m->ws, off) != hipSuccess) fail(SSB_ENOMEM, "hipMalloc of workspace failed");
  m->ws_bytes = off;
  char* wsb = static_cast<char*>(m->ws);
  m->h = reinterpret_cast<float*>(wsb + w_h);
  m->xg = wsb + w_xg;
  m->ssq = reinterpret_cast<float*>(wsb + w_ssq);
  m->q = wsb + w_q;
  m->attn = wsb + w_attn;
  m->act = wsb + w_act;
  m->row_tok = reinterpret_cast<int32_t*>(wsb + w_meta);
  m->row_pos = m->row_tok + MR;
  m->row_lim = m->row_pos + MR;
  m->row_req = m->row_lim + MR;
  m->row_slot = m->row_req + MR;
  m->row_cs = reinterpret_cast<float2*>(wsb + w_cs);
  m->part = reinterpret_cast<float*>(wsb + w_part);
  m->fwd_pt = reinterpret_cast<int32_t*>(wsb + w_fpt);
  m->am_tok = reinterpret_cast<int32_t*>(wsb + w_am);
  m->am_top1 = reinterpret_cast<float*>(m->am_tok + MR);
  m->am_top2 = m->am_top1 + MR;
  m->amv1 = reinterpret_cast<float*>(wsb + w_amp);
  m->amv2 = m->amv1 + (size_t)(lm_tiles / p_lm.NT) * MR;
  m->ami1 = reinterpret_cast<int32_t*>(m->amv2 + (size_t)(lm_tiles / p_lm.NT) * MR);
  m->ams = reinterpret_cast<float*>(wsb + w_ams);
  m->am_z = reinterpret_cast<float*>(wsb + w_conf);
  m->slog_d = m->sampling ? reinterpret_cast<float*>(wsb + w_slog) : nullptr;
  m->slog_v = m->sampling ? m->slog_d + (size_t)m->max_decode_rows * V : nullptr;
  m->smax_d = reinterpret_cast<float*>(wsb + w_sst);
  m->sz_d = m->smax_d + MR;
  m->smax_v = m->sz_d + MR;
  m->sz_v = m->smax_v + MR;
  m->dd_win = reinterpret_cast<int32_t*>(wsb + w_ddw);
  m->dd_rec = reinterpret_cast<int32_t*>(wsb + w_ddr);
  m->apart = reinterpret_cast<float*>(wsb + w_apart);
  m->accept_dev = reinterpret_cast<int32_t*>(wsb + w_acc);
  m->tok_dev = reinterpret_cast<int32_t*>(wsb + w_tok);
  m->req_dev = reinterpret_cast<ReqArgs*>(wsb + w_req);
  m->tail_sync = reinterpret_cast<unsigned long long*>(wsb + w_tail);
  m->tail_err = reinterpret_cast<int*>(wsb + w_tail + (size_t)kTailSyncWords * 8);
  hip_check(hipMemsetAsync(m->tail_sync, 0, (size_t)kTailSyncWords * 8 + 256, st), "clear layer-tail state");
  {
    // the fused layer tail needs one workgroup per CU for kTailWgs workgroups, and the GEMM plans it is
    // written for (O and down: one tile, 8 K slices of 4 and 16 steps; gate|up: two tiles, 4 slices of 8)
    int cus = 0;
    hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, m->device), "CU count");
    const GemmShape &o = m->o[0], &g = m->gu[0], &d = m->d[0];
    m->tail_ok = c.dtype == SSB_BF16 && cus >= kTailWgs && o.NT == 1 && o.KSL == 8 && o.S == 1 && o.K == 1024 &&
                 g.NT == 2 && g.KSL == 4 && g.K == 1024 && g.n_tiles == 2 * kTailWgs && d.NT == 1 && d.KSL == 8 &&
                 d.S == 1 && d.K == 4096 && o.n_tiles == d.n_tiles && o.n_tiles * 3 <= kTailWgs;
  }
  if (hipHostMalloc(reinterpret_cast<void**>(&m->req_pin), sizeof(ReqArgs), hipHostMallocDefault) != hipSuccess)
    fail(SSB_ENOMEM, "pinned host allocation failed");
  hip_check(hipStreamCreateWithFlags(&m->cap, hipStreamNonBlocking), "capture stream");
  if (hipHostMalloc(reinterpret_cast<void**>(&m->pin_i32), (size_t)(MR + kMaxReq * kOutStride) * 4,
                    hipHostMallocDefault) != hipSuccess)
    fail(SSB_ENOMEM, "pinned host allocation failed");
  if (hipHostMalloc(reinterpret_cast<void**>(&m->pin_f32), (size_t)2 * MR * 4, hipHostMallocDefault) !=
      hipSuccess)
    fail(SSB_ENOMEM, "pinned host allocation failed");
  hip_check(hipStreamSynchronize(st), "init sync");
  scratch_setup(m->device);
  *out = hold.release();
}

// ---------------------------------------------------------------------------
// Forward pass over a row set.
// ---------------------------------------------------------------------------
struct FwdSpec {
  int mode;           // PrepMode
  int M;              // rows
  int pos0;           // PREFILL / TOKENS
  const void* prefix; // PREFILL
  ReqArgs ra;         // host copy of the request state (already uploaded to the device)
  int max_pos;        // largest position of any row + 1
  int slots;          // graph capture: attention chunk slots of the launch (slot_bucket of max_pos)
  bool graph;         // launches are being captured: no round-dependent launch shapes
  float* logits;      // nullable [M][vocab] (all rows) or [1][vocab] (last row only)
  bool lm_last_only;  // LM head on the last row only (prefill)
  bool no_head;       // no LM head (cache-write forward)
  float stat_sc;      // > 0: row softmax sums at scale log2(e) / T (confidence: T = 1; sampling)
  bool sample;        // draw each window row's token from its distribution (needs logits, stat_sc)
  float* st_max;      // nullable: row max output (default: the greedy top-1 buffer)
  float* st_z;        // nullable: row exp-sum output (default: am_z)
};

template <typename T>
void forward(ssb_model* m, ssb_pool* pool, const FwdSpec& f, hipStream_t st) {
  const ssb_config& c = m->c;
  const int H = c.hidden, qd = c.n_heads * c.head_dim, MR = c.max_rows;
  const int M = f.M;
  const bool tall = f.mode == PREP_PREFILL || f.mode == PREP_TOKENS;
  // tall bf16 forwards use the large-tile GEMM (no decode row is computed there); its activations
  // (the GEMM inputs xg, attention output and SwiGLU output) are written and read fragment-major,
  // one contiguous 1 KiB block per matrix-core operand fragment; the last layer's xg stays
  // row-major for the LM head
  const bool big = tall && m->elem == 2 && M >= 128;
  const int pk = big ? 1 : 0;
  PrepArgs pa{};
  pa.mode = f.mode; pa.M = M; pa.hidden = H; pa.vocab = c.vocab; pa.mask_id = c.mask_id;
  pa.pos0 = f.pos0; pa.prefix = f.prefix; pa.tokens = m->tok_dev; pa.am_prev = m->am_tok;
  pa.embed = m->embed; pa.gain = m->attn_norm[0];
  pa.row_tok = m->row_tok; pa.row_pos = m->row_pos; pa.row_lim = m->row_lim; pa.row_req = m->row_req;
  pa.row_slot = m->row_slot; pa.row_cs = m->row_cs; pa.rope = m->rope; pa.half = c.head_dim / 2;
  pa.fwd_pt = m->fwd_pt; pa.pt_ld = m->pt_ld;
  pa.h = m->h; pa.xg = m->xg; pa.ssq = m->ssq; pa.ssq_ld = H / 16; pa.req = m->req_dev; pa.xpk = pk;
  pa.stamp = prof_begin(m, kKindPrep, st);
  hip_check(launch_prep<T>(pa, st), "prep");
  prof_end(m, kKindPrep, st);

  GemmArgs g{};
  g.M = M;
  g.ssq = m->ssq; g.ssq_ld = H / 16; g.n_ssq = H / 16; g.eps = c.rms_eps; g.hidden = H;
  g.h = m->h; g.xg_out = m->xg; g.ssq_out = m->ssq;
  g.q = m->q; g.q_ld = qd;
  g.n_heads = c.n_heads; g.n_kv = c.n_kv_heads; g.head_dim = c.head_dim; g.n_pages = pool->n_pages;
  g.kv_pool = pool->base; g.row_slot = m->row_slot; g.row_cs = m->row_cs;
  g.part = m->part; g.part_ld = H;
  g.act = m->act; g.act_ld = c.ffn;
  g.vocab = c.vocab; g.mask_id = c.mask_id;
  auto set_w = [](GemmArgs& a, const GemmShape& s) {
    a.W = s.W; a.K = s.K; a.n_tiles = s.n_tiles; a.NT = s.NT; a.KSL = s.KSL; a.S = s.S;
  };

  AttnArgs at{};
  at.q = m->q; at.q_ld = qd; at.kv_pool = pool->base; at.n_pages = pool->n_pages;
  at.n_heads = c.n_heads; at.n_kv = c.n_kv_heads;
  at.req = m->req_dev;
  at.fwd_pt = m->fwd_pt; at.pt_ld = m->pt_ld;
  at.row_lim = m->row_lim; at.part = m->apart; at.max_chunks = m->max_chunks;
  at.out = m->attn; at.out_ld = qd;
  // rows of a prefill or teacher-forced forward fold their key chunks in one workgroup (no
  // records, no combine launch); decode windows split keys over workgroups and combine
  at.fold = (tall || M > m->max_decode_rows) ? 1 : 0;
  at.opk = pk;
  // decode forwards of many rows (batched rounds) use the large-tile GEMM's exact form, which
  // reproduces k_gemm's arithmetic bit for bit (k_gemm keeps the small-M shapes it is fast at)
  const bool dec_big = !tall && m->elem == 2;
  const bool x_qkv = dec_big && M >= kExactRowsQkv, x_o = dec_big && M >= kExactRowsO;
  const bool x_gu = dec_big && M >= kExactRowsGateUp, x_down = dec_big && M >= kExactRowsDown;
  at.scale = 1.0f / std::sqrt((float)c.head_dim);
  // row tasks: windows of each request (draft/verify) or one request's rows
  at.tasks.n = 0;
  // row tasks; window tasks read their largest visibility limit (p + B, or
  // p + B + 1 for verify) from the device request state
  auto add_tasks = [&](int req, int row0, int nrows, int lim_mode, int last_pos) {
    for (int r = 0; r < nrows; r += kTaskRows) {
      if (at.tasks.n >= kMaxTasks) fail(SSB_EINVAL, "too many attention row tasks");
      const int n = std::min(kTaskRows, nrows - r);
      at.tasks.t[at.tasks.n++] = AttnTask{req, row0 + r, n, last_pos < 0 ? -1 : last_pos - (nrows - r - n), lim_mode};
    }
  };
  if (f.mode == PREP_DRAFT || f.mode == PREP_VERIFY) {
    for (int r = 0; r < f.ra.n; ++r) add_tasks(r, f.ra.row0[r], f.ra.B + 1, f.mode == PREP_DRAFT ? 1 : 2, -1);
  } else {
    add_tasks(0, 0, M, 0, f.pos0 + M - 1);
  }
  const int chunk_slots = f.graph ? (f.slots > 0 ? f.slots : m->max_chunks) : (f.max_pos - 1) / kKeyChunk + 1;
  // decode windows of at most 48 rows run each layer's O, gate|up and down as one fused launch
  // (same per-row arithmetic as the three GEMM launches); forwards without an LM head keep the
  // three launches, since the argmax is what reports a failed layer-tail barrier
  const bool tail = m->tail_ok && !m->no_fused && !tall && M <= 48 && !f.no_head;

  for (int l = 0; l < c.n_layers; ++l) {
    g.layer = l;
    {  // RMSNorm -> QKV -> RoPE -> KV write (input xg = h * attn_norm[l])
      GemmArgs a = g;
      set_w(a, m->qkv[l]);
      a.x = m->xg; a.ldx = H; a.xpk = pk;
      a.stamp = prof_begin(m, SSB_K_QKV, st);
      hip_check(big || x_qkv ? launch_gemm_big(a, EPI_QKV, x_qkv, st) : launch_gemm<T>(a, EPI_QKV, st), "qkv gemm");
      prof_end(m, SSB_K_QKV, st);
    }
    at.layer = l;
    at.stamp = prof_begin(m, SSB_K_ATTN, st);
    hip_check(launch_attn<T>(at, chunk_slots, c.head_dim, st), "attention");
    prof_end(m, SSB_K_ATTN, st);
    if (!at.fold) {
      ProfStamp* cst = prof_begin(m, SSB_K_COMBINE, st);
      hip_check(launch_attn_combine<T>(m->apart, m->max_chunks, chunk_slots, c.n_heads, c.head_dim, m->row_lim, M,
                                       m->attn, qd, st, cst), "attention combine");
      prof_end(m, SSB_K_COMBINE, st);
    }
    if (tail) {  // O + residual, gate|up + SwiGLU, down + residual in one launch
      TailArgs ta{};
      ta.o = g; set_w(ta.o, m->o[l]); ta.o.x = m->attn; ta.o.ldx = qd; ta.o.gain_next = m->mlp_norm[l];
      ta.gu = g; set_w(ta.gu, m->gu[l]); ta.gu.x = m->xg; ta.gu.ldx = H;
      ta.d = g; set_w(ta.d, m->d[l]); ta.d.x = m->act; ta.d.ldx = c.ffn;
      ta.d.gain_next = l + 1 < c.n_layers ? m->attn_norm[l + 1] : m->final_norm;
      ta.sync = m->tail_sync;
      ta.err = m->tail_err;
      ta.stamp = prof_begin(m, SSB_K_TAIL, st);
      hip_check(launch_layer_tail(ta, st), "layer tail");
      prof_end(m, SSB_K_TAIL, st);
      continue;
    }
    {  // O + residual; next input xg = h * mlp_norm[l]
      GemmArgs a = g;
      set_w(a, m->o[l]);
      a.x = m->attn; a.ldx = qd; a.xpk = pk; a.opk = pk;
      a.gain_next = m->mlp_norm[l];
      a.stamp = prof_begin(m, SSB_K_O, st);
      hip_check(big || x_o ? launch_gemm_big(a, EPI_RESID, x_o, st) : launch_gemm<T>(a, EPI_RESID, st), "o gemm");
      prof_end(m, SSB_K_O, st);
    }
    {  // gate|up + SwiGLU
      GemmArgs a = g;
      set_w(a, m->gu[l]);
      a.x = m->xg; a.ldx = H; a.xpk = pk; a.opk = pk;
      a.stamp = prof_begin(m, SSB_K_GATEUP, st);
      hip_check(big || x_gu ? launch_gemm_big(a, EPI_SWIGLU, x_gu, st) : launch_gemm<T>(a, EPI_SWIGLU, st),
                "gate/up gemm");
      prof_end(m, SSB_K_GATEUP, st);
    }
    {  // down + residual; next input xg = h * (next attn_norm | final_norm)
      GemmArgs a = g;
      set_w(a, m->d[l]);
      a.x = m->act; a.ldx = c.ffn; a.xpk = pk; a.opk = l + 1 < c.n_layers ? pk : 0;
      a.gain_next = l + 1 < c.n_layers ? m->attn_norm[l + 1] : m->final_norm;
      a.stamp = prof_begin(m, SSB_K_DOWN, st);
      const bool dexact = x_down && a.S == 1;   // a K-split down projection stays on k_gemm
      if (big || dexact) hip_check(launch_gemm_big(a, EPI_RESID, dexact, st), "down gemm");
      else hip_check(launch_gemm<T>(a, a.S > 1 ? EPI_PARTIAL : EPI_RESID, st), "down gemm");
      prof_end(m, SSB_K_DOWN, st);
      if (a.S > 1 && !big) {
        a.stamp = prof_begin(m, SSB_K_REDUCE, st);
        hip_check(launch_resid_reduce<T>(a, st), "down reduce");
        prof_end(m, SSB_K_REDUCE, st);
      }
    }
  }
  // LM head + argmax
  if (!f.no_head) {
    GemmArgs a = g;
    set_w(a, m->lm);
    a.x = m->xg; a.ldx = H;
    a.logits = f.logits;
    const int n_groups = m->lm.n_tiles / m->lm.NT;
    a.am_v1 = m->amv1; a.am_i1 = m->ami1; a.am_v2 = m->amv2; a.am_ld = n_groups;
    a.am_s = f.stat_sc > 0.f ? m->ams : nullptr;
    a.am_scale = f.stat_sc;
    int rows = M;
    if (f.lm_last_only) {
      a.x = reinterpret_cast<const char*>(m->xg) + (size_t)(M - 1) * H * m->elem;
      a.ssq = m->ssq + (size_t)(M - 1) * (H / 16);
      a.M = 1;
      rows = 1;
    }
    a.stamp = prof_begin(m, SSB_K_LMHEAD, st);
    const bool x_lm = dec_big && rows >= kExactRowsLm && !a.am_s && a.NT == 4 && a.n_tiles % 8 == 0;
    if (x_lm) hip_check(launch_gemm_big(a, EPI_LOGITS, true, st), "lm head gemm");
    else hip_check(launch_gemm<T>(a, EPI_LOGITS, st), "lm head gemm");
    prof_end(m, SSB_K_LMHEAD, st);
    ProfStamp* ast = prof_begin(m, SSB_K_ARGMAX, st);
    float* top1 = f.st_max ? f.st_max : m->am_top1;
    float* zs = f.st_z ? f.st_z : m->am_z;
    hip_check(launch_argmax(m->amv1, m->ami1, m->amv2, f.stat_sc > 0.f ? m->ams : nullptr, f.stat_sc, n_groups,
                            n_groups, rows, m->am_tok, top1, m->am_top2, zs, st, ast, m->tail_err), "argmax");
    prof_end(m, SSB_K_ARGMAX, st);
    if (f.sample) {
      if (!f.logits || !(f.stat_sc > 0.f)) fail(SSB_EINVAL, "sampling needs logits and row sums");
      SampleArgs sa{};
      sa.v1 = m->amv1; sa.gs = m->ams; sa.ld = n_groups; sa.n_groups = n_groups; sa.gcols = m->lm.NT * 16;
      sa.logits = f.logits; sa.vocab = c.vocab; sa.mask_id = c.mask_id;
      sa.rmax = top1; sa.rz = zs; sa.sc = f.stat_sc; sa.req = m->req_dev; sa.tok = m->am_tok;
      const bool win = f.mode == PREP_DRAFT || f.mode == PREP_VERIFY;
      hip_check(launch_sample_rows(sa, win ? f.ra.B + 1 : 1, win ? f.ra.n : 1, st), "sample rows");
    }
  }
}

void run_forward(ssb_model* m, ssb_pool* pool, const FwdSpec& f, hipStream_t st) {
  if (m->c.dtype == SSB_BF16) forward<bf16_t>(m, pool, f, st);
  else forward<float>(m, pool, f, st);
}

// ---------------------------------------------------------------------------
// KV pages
// ---------------------------------------------------------------------------
// Pages for positions [0, n_tokens), new page ids uploaded to the device table (stream-ordered).
void kv_ensure(ssb_kv* kv, int n_tokens, hipStream_t st) {
  const int first = kv->ensure(*kv->pool, n_tokens, kv->pt_host);
  const int need = (int)kv->pages.size();
  if (need > first)
    hip_check(hipMemcpyAsync(kv->pt_dev + first, kv->pt_host + first, (size_t)(need - first) * 4,
                             hipMemcpyHostToDevice, st), "page table upload");
}

// Return pages wholly at positions >= keep_tokens.
void kv_trim(ssb_kv* kv, int keep_tokens) { kv->trim(*kv->pool, keep_tokens); }

ssb_kv* kv_new(ssb_pool* p, int max_tokens) {
  if (max_tokens > p->m->c.max_positions) fail(SSB_EINVAL, "max_tokens exceeds max_positions");
  hip_check(hipSetDevice(p->m->device), "hipSetDevice");
  auto* kv = new ssb_kv();
  std::unique_ptr<ssb_kv> hold(kv);
  kv->pool = p;
  kv->init(max_tokens);
  if (hipMalloc(reinterpret_cast<void**>(&kv->pt_dev), (size_t)kv->max_pages * 4) != hipSuccess)
    fail(SSB_ENOMEM, "page table allocation failed");
  if (hipHostMalloc(reinterpret_cast<void**>(&kv->pt_host), (size_t)kv->max_pages * 4, hipHostMallocDefault) !=
      hipSuccess) {
    (void)hipFree(kv->pt_dev);
    fail(SSB_ENOMEM, "pinned page table allocation failed");
  }
  return hold.release();
}

void kv_delete(ssb_kv* kv) {
  if (!kv) return;
  (void)hipSetDevice(kv->pool->m->device);
  (void)hipDeviceSynchronize();
  kv_trim(kv, 0);
  (void)hipFree(kv->pt_dev);
  (void)hipHostFree(kv->pt_host);
  delete kv;
}

hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }


void check_model_kv(ssb_model* m, ssb_kv* kv) {
  if (!m) fail(SSB_EINVAL, "null model");
  if (!kv) fail(SSB_EINVAL, "null kv");
  if (kv->pool->m != m) fail(SSB_EINVAL, "kv belongs to another model");
  hip_check(hipSetDevice(m->device), "hipSetDevice");
}

// Copies the request state to the device (stream-ordered before the launches
// that read it).  The pinned staging buffer is reused: every ABI call
// synchronizes its stream before returning.
void upload_req(ssb_model* m, const ReqArgs& ra, hipStream_t st) {
  *m->req_pin = ra;
  hip_check(hipMemcpyAsync(m->req_dev, m->req_pin, sizeof(ReqArgs), hipMemcpyHostToDevice, st),
            "upload request state");
}

// Graph of a fixed launch sequence, captured once per (kind, pool, R, B) on a
// private stream and replayed on the caller's stream.  Launch shapes inside
// never depend on the round; round state is read from the device.
// Attention chunk slots a captured launch covers for windows ending before max_pos: the chunk
// count rounded up to a multiple of 8 (so a growing sequence re-captures once per 512 positions),
// at most the model's chunk capacity.  Slots past a window's last chunk exit at once.
int slot_bucket(const ssb_model* m, int max_pos) {
  const int c = (max_pos - 1) / kKeyChunk + 1;
  return std::min((c + 7) / 8 * 8, m->max_chunks);
}

hipGraphExec_t get_graph(ssb_model* m, int kind, ssb_pool* pool, int R, int B, int slots,
                         const std::function<void(hipStream_t)>& body, float temperature = 0.f) {
  uint32_t tb = 0;
  std::memcpy(&tb, &temperature, 4);
  // a graph that times one kernel kind (stamps in every launch) is kept apart
  const int pk = m->prof_graph ? m->prof_kind + 1 : 0;
  const auto key = std::make_tuple(kind * 64 + pk, static_cast<void*>(pool), R, B, tb, slots);
  auto it = m->graphs.find(key);
  if (it != m->graphs.end()) {
    if (pk) {   // read back after the replay
      m->prof_cap_kinds = m->graph_prof_kinds[it->second];
      m->prof_stamp_used = (int)m->prof_cap_kinds.size();
    }
    return it->second;
  }
  m->prof_stamp_used = 0;
  m->prof_cap_kinds.clear();
  m->capturing = true;
  hip_check(hipStreamBeginCapture(m->cap, hipStreamCaptureModeThreadLocal), "begin capture");
  try {
    body(m->cap);
  } catch (...) {
    m->capturing = false;
    m->prof_stamp_used = 0;
    hipGraph_t tmp = nullptr;
    (void)hipStreamEndCapture(m->cap, &tmp);
    if (tmp) (void)hipGraphDestroy(tmp);
    throw;
  }
  m->capturing = false;
  hipGraph_t g = nullptr;
  hip_check(hipStreamEndCapture(m->cap, &g), "end capture");
  hipGraphExec_t ex = nullptr;
  const hipError_t e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  hip_check(e, "graph instantiate");
  m->graphs[key] = ex;
  if (pk) m->graph_prof_kinds[ex] = m->prof_cap_kinds;   // slots written by each replay
  else m->prof_stamp_used = 0;
  return ex;
}

ReqArgs single_req(ssb_kv* kv, int B, int max_commit) {
  ReqArgs ra{};
  ra.n = 1;
  ra.B = B;
  ra.p[0] = kv->seq_len;
  ra.x0[0] = kv->x0;
  ra.row0[0] = 0;
  ra.max_commit[0] = max_commit;
  ra.pt[0] = kv->pt_dev;
  ra.npg[0] = (int)kv->pages.size();
  return ra;
}

// Sampling variant of a call: temperature and, per request, its device uniforms.
struct SampleSpec {
  float temperature;
  const float* const* u;
};

void check_sample(const ssb_model* m, const SampleSpec* smp, int R) {
  if (!smp) return;
  if (!m->sampling) fail(SSB_EINVAL, "the model was initialised without SSB_FEAT_SAMPLE");
  if (!(smp->temperature > 0.f) || !(smp->temperature < INFINITY)) fail(SSB_EINVAL, "temperature must be > 0");
  for (int r = 0; r < R; ++r)
    if (!smp->u[r]) fail(SSB_EINVAL, "null uniforms");
}

void prefill(ssb_model* m, ssb_kv* kv, const void* prefix, int P, int32_t* first, hipStream_t st,
             const SampleSpec* smp = nullptr) {
  check_model_kv(m, kv);
  if (!prefix) fail(SSB_EINVAL, "null prefix");
  if (P < 1) fail(SSB_EINVAL, "P must be >= 1");
  if (kv->seq_len != 0 || kv->x0 >= 0) fail(SSB_ESTATE, "prefill needs an empty kv");
  if (P + 1 > m->c.max_positions) fail(SSB_EINVAL, "P exceeds max_positions");
  check_sample(m, smp, 1);
  kv_ensure(kv, P, st);
  ReqArgs ra = single_req(kv, 0, 1);
  if (smp) ra.u[0] = smp->u[0];
  upload_req(m, ra, st);
  for (int p0 = 0; p0 < P; p0 += m->c.max_rows) {
    FwdSpec f{};
    f.mode = PREP_PREFILL;
    f.M = std::min(m->c.max_rows, P - p0);
    f.pos0 = p0;
    f.prefix = prefix;
    f.ra = ra;
    f.max_pos = p0 + f.M;
    f.lm_last_only = true;
    if (smp && p0 + f.M == P) {   // y1 drawn from the last row's distribution
      f.logits = m->slog_d;
      f.stat_sc = kLog2e / smp->temperature;
      f.sample = true;
    }
    run_forward(m, kv->pool, f, st);
  }
  hip_check(hipMemcpyAsync(m->pin_i32, m->am_tok, 4, hipMemcpyDeviceToHost, st), "copy token");
  hip_check(hipStreamSynchronize(st), "prefill sync");
  prof_collect(m);
  const int32_t y1 = m->pin_i32[0];
  if (y1 < 0 || y1 >= m->c.vocab) fail(SSB_EHIP, "prefill produced no valid token (NaN logits?)");
  kv->seq_len = P;
  kv->x0 = y1;
  if (first) *first = y1;
}

// Runs draft + verify + accept for R requests (row windows concatenated).
// Debug: NaN into the KV slots [lo, p + B + 2) of every request of the launch (lo = p + 1 with no
// accept record, p + A + 2 with one).
void poison_kv(ssb_model* m, ssb_pool* pool, int R, const int32_t* acc, hipStream_t s, int lo = -1, int hi = -1) {
  const ssb_config& c = m->c;
  if (m->elem == 2)
    hip_check(launch_poison_kv<bf16_t>(m->req_dev, R, acc, kOutStride, lo, hi, pool->base, c.n_layers, pool->n_pages,
                                       c.n_kv_heads, c.head_dim, s), "poison kv");
  else
    hip_check(launch_poison_kv<float>(m->req_dev, R, acc, kOutStride, lo, hi, pool->base, c.n_layers, pool->n_pages,
                                      c.n_kv_heads, c.head_dim, s), "poison kv");
}

void round_impl(ssb_model* m, ssb_kv* const* kvs, int R, int B, const int* max_commit, const int32_t* planted,
                const int32_t* const* cont, const int* cont_len, const int* cont_c, const int* astar,
                float* dlog, float* vlog, RoundOut* out, hipStream_t st, const SampleSpec* smp = nullptr) {
  const ssb_config& c = m->c;
  check_sample(m, smp, R);
  if (smp && (planted || cont)) fail(SSB_EINVAL, "planted drafts apply to greedy rounds only");
  if (R < 1 || R > m->max_batch) fail(SSB_EINVAL, "R must be in [1, max_batch]");
  if (B < 0 || B > c.block_B) fail(SSB_EINVAL, "B must be in [0, block_B]");
  if (R * (B + 1) > c.max_rows) fail(SSB_EINVAL, "R*(B+1) exceeds max_rows");
  ssb_pool* pool = kvs[0]->pool;
  for (int r = 0; r < R; ++r) {
    check_model_kv(m, kvs[r]);
    if (kvs[r]->pool != pool) fail(SSB_EINVAL, "batched kvs must share one pool");
    if (kvs[r]->x0 < 0) fail(SSB_ESTATE, "round needs a prefilled kv (no boundary token)");
    if (max_commit[r] < 1) fail(SSB_EINVAL, "max_commit must be >= 1");
    if (kvs[r]->seq_len + B + 2 > c.max_positions) fail(SSB_ENOKV, "window exceeds max_positions");
    for (int q = 0; q < r; ++q)
      if (kvs[q] == kvs[r]) fail(SSB_EINVAL, "the same kv appears twice in a batch");
  }
  for (int r = 0; r < R; ++r) kv_ensure(kvs[r], kvs[r]->seq_len + B + 2, st);
  ReqArgs ra{};
  ra.n = R;
  ra.B = B;
  int maxpos = 0;
  for (int r = 0; r < R; ++r) {
    ra.p[r] = kvs[r]->seq_len;
    ra.x0[r] = kvs[r]->x0;
    ra.row0[r] = r * (B + 1);
    ra.max_commit[r] = max_commit[r];
    ra.pt[r] = kvs[r]->pt_dev;
    ra.npg[r] = (int)kvs[r]->pages.size();
    ra.planted[r] = planted ? planted + (size_t)r * B : nullptr;
    ra.cont[r] = cont ? cont[r] : nullptr;
    ra.cont_len[r] = cont_len ? cont_len[r] : 0;
    ra.cont_c[r] = cont_c ? cont_c[r] : 0;
    ra.astar[r] = astar ? astar[r] : 0;
    ra.u[r] = smp ? smp->u[r] : nullptr;
    maxpos = std::max(maxpos, ra.p[r] + B + 2);
  }
  upload_req(m, ra, st);
  const int slots = slot_bucket(m, maxpos);
  auto body = [&](hipStream_t s, bool graph) {
    FwdSpec f{};
    f.M = R * (B + 1);
    f.ra = ra;
    f.max_pos = maxpos;
    f.slots = slots;
    f.graph = graph;
    f.mode = PREP_DRAFT;
    f.logits = dlog;
    if (smp) {
      // stochastic round: every draft row drawn from its distribution (a0, d_1..d_B)
      f.logits = dlog ? dlog : m->slog_d;
      f.stat_sc = kLog2e / smp->temperature;
      f.sample = true;
      f.st_max = m->smax_d;
      f.st_z = m->sz_d;
    }
    run_forward(m, pool, f, s);
    if (m->debug_poison) poison_kv(m, pool, R, nullptr, s);   // the window slots verify rewrites
    f.mode = PREP_VERIFY;
    f.logits = vlog;
    if (smp) {
      f.logits = vlog ? vlog : m->slog_v;
      f.sample = false;
      f.st_max = m->smax_v;
      f.st_z = m->sz_v;
    }
    run_forward(m, pool, f, s);
    if (smp) {
      AcceptSampleArgs aa{};
      aa.row_tok = m->row_tok;
      aa.lg_d = dlog ? dlog : m->slog_d; aa.dmax = m->smax_d; aa.dz = m->sz_d;
      aa.lg_v = vlog ? vlog : m->slog_v; aa.vmax = m->smax_v; aa.vz = m->sz_v;
      aa.vocab = c.vocab; aa.mask_id = c.mask_id; aa.eos_id = c.eos_id; aa.sc = kLog2e / smp->temperature;
      aa.req = m->req_dev; aa.out = m->accept_dev; aa.out_stride = kOutStride; aa.err = m->tail_err;
      hip_check(launch_accept_sample(aa, R, s), "stochastic accept");
    } else {
      ProfStamp* ast = prof_begin(m, kKindAccept, s);
      hip_check(launch_accept(m->row_tok, m->am_tok, m->req_dev, R, c.eos_id, m->accept_dev, kOutStride, s,
                              m->tail_err, ast),
                "accept");
      prof_end(m, kKindAccept, s);
    }
    if (m->debug_poison) poison_kv(m, pool, R, m->accept_dev, s);   // the rolled-back slots
    hip_check(hipMemcpyAsync(m->pin_i32, m->accept_dev, (size_t)R * kOutStride * 4, hipMemcpyDeviceToHost, s),
              "copy accept");
  };
  if (dlog || vlog || prof_eager(m) || m->debug_poison || m->no_graph) {
    body(st, false);
  } else {
    hipGraphExec_t ex = get_graph(m, smp ? 4 : 0, pool, R, B, slots, [&](hipStream_t s) { body(s, true); },
                                  smp ? smp->temperature : 0.f);
    hip_check(hipGraphLaunch(ex, st), "round graph launch");
  }
  hip_check(hipStreamSynchronize(st), "round sync");
  prof_collect(m);
  commit_batch(kvs, R, *pool, ra.p, m->pin_i32, B, c.vocab, c.mask_id, out);
}

void ar_step(ssb_model* m, ssb_kv* kv, int32_t* token, float* logits, hipStream_t st,
             const SampleSpec* smp = nullptr) {
  check_model_kv(m, kv);
  check_sample(m, smp, 1);
  if (kv->x0 < 0) fail(SSB_ESTATE, "AR step needs a prefilled kv (no boundary token)");
  if (kv->seq_len + 1 > m->c.max_positions) fail(SSB_ENOKV, "position exceeds max_positions");
  kv_ensure(kv, kv->seq_len + 1, st);
  // an AR step is a draft window with no masks: [x0] at p, keys <= p
  ReqArgs ra = single_req(kv, 0, 1);
  if (smp) ra.u[0] = smp->u[0];
  upload_req(m, ra, st);
  auto body = [&](hipStream_t s, bool graph) {
    FwdSpec f{};
    f.mode = PREP_DRAFT;
    f.M = 1;
    f.ra = ra;
    f.max_pos = kv->seq_len + 1;
    f.slots = slot_bucket(m, f.max_pos);
    f.graph = graph;
    f.logits = logits;
    if (smp) {
      f.logits = logits ? logits : m->slog_d;
      f.stat_sc = kLog2e / smp->temperature;
      f.sample = true;
    }
    run_forward(m, kv->pool, f, s);
    hip_check(hipMemcpyAsync(m->pin_i32, m->am_tok, 4, hipMemcpyDeviceToHost, s), "copy token");
  };
  if (logits || prof_eager(m)) {
    body(st, false);
  } else {
    hipGraphExec_t ex = get_graph(m, smp ? 5 : 1, kv->pool, 1, 0, slot_bucket(m, kv->seq_len + 1),
                                  [&](hipStream_t s) { body(s, true); },
                                  smp ? smp->temperature : 0.f);
    hip_check(hipGraphLaunch(ex, st), "AR graph launch");
  }
  hip_check(hipStreamSynchronize(st), "ar sync");
  prof_collect(m);
  const int32_t y = m->pin_i32[0];
  if (y < 0 || y >= m->c.vocab) fail(SSB_EHIP, "AR step produced no valid token (NaN logits?)");
  kv->seq_len += 1;
  kv->x0 = y;
  if (token) *token = y;
}

double now_us() {
  return std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// One greedy AR step for R requests, one launch per stage: request r's row is
// [x0_r] at p_r, keys <= p_r (the window of a round with no masks).
void ar_step_batch_impl(ssb_model* m, ssb_kv* const* kvs, int R, int32_t* tokens, hipStream_t st) {
  const ssb_config& c = m->c;
  if (R < 1 || R > m->max_batch) fail(SSB_EINVAL, "R must be in [1, max_batch]");
  if (R > c.max_rows) fail(SSB_EINVAL, "R exceeds max_rows");
  ssb_pool* pool = kvs[0]->pool;
  for (int r = 0; r < R; ++r) {
    check_model_kv(m, kvs[r]);
    if (kvs[r]->pool != pool) fail(SSB_EINVAL, "batched kvs must share one pool");
    if (kvs[r]->x0 < 0) fail(SSB_ESTATE, "AR step needs a prefilled kv (no boundary token)");
    if (kvs[r]->seq_len + 1 > c.max_positions) fail(SSB_ENOKV, "position exceeds max_positions");
    for (int q = 0; q < r; ++q)
      if (kvs[q] == kvs[r]) fail(SSB_EINVAL, "the same kv appears twice in a batch");
  }
  for (int r = 0; r < R; ++r) kv_ensure(kvs[r], kvs[r]->seq_len + 1, st);
  ReqArgs ra{};
  ra.n = R;
  ra.B = 0;
  int maxpos = 0;
  for (int r = 0; r < R; ++r) {
    ra.p[r] = kvs[r]->seq_len;
    ra.x0[r] = kvs[r]->x0;
    ra.row0[r] = r;
    ra.max_commit[r] = 1;
    ra.pt[r] = kvs[r]->pt_dev;
    ra.npg[r] = (int)kvs[r]->pages.size();
    maxpos = std::max(maxpos, ra.p[r] + 1);
  }
  upload_req(m, ra, st);
  auto body = [&](hipStream_t s, bool graph) {
    FwdSpec f{};
    f.mode = PREP_DRAFT;
    f.M = R;
    f.ra = ra;
    f.max_pos = maxpos;
    f.slots = slot_bucket(m, maxpos);
    f.graph = graph;
    run_forward(m, pool, f, s);
    hip_check(hipMemcpyAsync(m->pin_i32, m->am_tok, (size_t)R * 4, hipMemcpyDeviceToHost, s), "copy tokens");
  };
  if (prof_eager(m)) {
    body(st, false);
  } else {
    hipGraphExec_t ex = get_graph(m, 1, pool, R, 0, slot_bucket(m, maxpos), [&](hipStream_t s) { body(s, true); });
    hip_check(hipGraphLaunch(ex, st), "AR graph launch");
  }
  hip_check(hipStreamSynchronize(st), "ar sync");
  prof_collect(m);
  for (int r = 0; r < R; ++r) {
    const int32_t y = m->pin_i32[r];
    if (y < 0 || y >= c.vocab) fail(SSB_EHIP, "AR step produced no valid token (NaN logits?)");
    tokens[r] = y;
  }
  for (int r = 0; r < R; ++r) {
    kvs[r]->seq_len += 1;
    kvs[r]->x0 = tokens[r];
  }
}

// Continuous batching over a queue of requests, all present at the start
// (the batch-size throughput setting of the GravityOCR review, section 4.3 /
// Figure 6: a full client queue and a cap on running requests).  Up to
// max_running requests run at once; a free slot admits the next request in
// queue order (its prefill runs between decode launches); every decode launch
// advances all running requests by one greedy AR step or one round; a request
// leaves at EOS or its max_len.
void serve_impl(ssb_model* m, ssb_pool* pool, ssb_request* reqs, int n_reqs, int max_running, int mode, int B,
                int max_tokens, ssb_serve_stats* stats, hipStream_t st) {
  const ssb_config& c = m->c;
  if (!pool || pool->m != m) fail(SSB_EINVAL, "pool belongs to another model");
  if (n_reqs < 0 || (n_reqs > 0 && !reqs)) fail(SSB_EINVAL, "bad request array");
  if (mode != SSB_SERVE_AR && mode != SSB_SERVE_SPEC) fail(SSB_EINVAL, "unknown serve mode");
  if (max_running < 1 || max_running > m->max_batch) fail(SSB_EINVAL, "max_running must be in [1, max_batch]");
  if (mode == SSB_SERVE_SPEC) {
    if (B < 0 || B > c.block_B) fail(SSB_EINVAL, "B must be in [0, block_B]");
    if (max_running * (B + 1) > c.max_rows) fail(SSB_EINVAL, "max_running * (B + 1) exceeds max_rows");
  } else if (max_running > c.max_rows) {
    fail(SSB_EINVAL, "max_running exceeds max_rows");
  }
  const int W = mode == SSB_SERVE_SPEC ? B + 2 : 1;
  for (int i = 0; i < n_reqs; ++i) {
    const ssb_request& q = reqs[i];
    if (!q.prefix_dev || q.P < 1 || q.max_len < 0 || (q.max_len > 0 && !q.out))
      fail(SSB_EINVAL, "bad request " + std::to_string(i));
    if (q.P + q.max_len + W + 1 > max_tokens) fail(SSB_EINVAL, "request exceeds max_tokens");
    if (q.cont_dev && (q.cont_len < 0 || (q.n_astar > 0 && !q.astar))) fail(SSB_EINVAL, "bad planting");
  }
  struct Slot { ssb_kv* kv = nullptr; int req = -1, k = 0, n = 0; };
  std::vector<Slot> slots(max_running);
  struct Hold {
    std::vector<Slot>& s;
    ~Hold() { for (auto& x : s) kv_delete(x.kv); }
  } hold{slots};
  for (auto& x : slots) x.kv = kv_new(pool, max_tokens);
  ssb_serve_stats S0{};
  const double t0 = now_us();
  int next = 0;
  double running_sum = 0;
  auto finish = [&](Slot& x) {
    ssb_request& q = reqs[x.req];
    q.n_out = x.n;
    q.rounds = x.k;
    q.finish_us = now_us() - t0;
    S0.tokens += x.n;
    x.req = -1;
  };
  std::vector<ssb_kv*> kvs;
  std::vector<Slot*> run;
  std::vector<int32_t> toks;
  std::vector<int> mc, cl, cc, as;
  std::vector<const int32_t*> conts;
  std::vector<RoundOut> outs;
  for (;;) {
    for (auto& x : slots) {
      while (x.req < 0 && next < n_reqs) {
        x.req = next++;
        x.k = 0;
        x.n = 0;
        ssb_request& q = reqs[x.req];
        if (q.max_len == 0) { finish(x); continue; }
        kv_trim(x.kv, 0);
        x.kv->seq_len = 0;
        x.kv->x0 = -1;
        const double tp = now_us();
        int32_t y1 = 0;
        prefill(m, x.kv, q.prefix_dev, q.P, &y1, st);
        S0.prefill_us += now_us() - tp;
        S0.prefills += 1;
        q.out[x.n++] = y1;
        if (y1 == c.eos_id || x.n >= q.max_len) finish(x);
      }
    }
    run.clear();
    kvs.clear();
    for (auto& x : slots)
      if (x.req >= 0) { run.push_back(&x); kvs.push_back(x.kv); }
    if (run.empty()) break;
    const int R = (int)run.size();
    const double td = now_us();
    if (mode == SSB_SERVE_AR) {
      toks.assign(R, 0);
      ar_step_batch_impl(m, kvs.data(), R, toks.data(), st);
      for (int r = 0; r < R; ++r) {
        Slot& x = *run[r];
        ssb_request& q = reqs[x.req];
        q.out[x.n++] = toks[r];
        x.k += 1;
        if (toks[r] == c.eos_id || x.n >= q.max_len) finish(x);
      }
    } else {
      mc.assign(R, 0); cl.assign(R, 0); cc.assign(R, 0); as.assign(R, 0);
      conts.assign(R, nullptr);
      outs.assign(R, RoundOut{});
      bool any_plant = false;
      for (int r = 0; r < R; ++r) {
        const Slot& x = *run[r];
        const ssb_request& q = reqs[x.req];
        mc[r] = q.max_len - x.n;
        if (q.cont_dev && x.k < q.n_astar) {
          conts[r] = q.cont_dev;
          cl[r] = q.cont_len;
          cc[r] = x.n;
          as[r] = q.astar[x.k];
          any_plant = true;
        }
      }
      round_impl(m, kvs.data(), R, B, mc.data(), nullptr, any_plant ? conts.data() : nullptr, cl.data(), cc.data(),
                 as.data(), nullptr, nullptr, outs.data(), st);
      for (int r = 0; r < R; ++r) {
        Slot& x = *run[r];
        ssb_request& q = reqs[x.req];
        for (int i = 0; i < outs[r].n; ++i) q.out[x.n++] = outs[r].tok[i];
        x.k += 1;
        if (outs[r].eos || x.n >= q.max_len) finish(x);
      }
    }
    S0.decode_us += now_us() - td;
    S0.steps += 1;
    running_sum += R;
  }
  S0.total_us = now_us() - t0;
  S0.mean_running = S0.steps ? running_sum / S0.steps : 0.0;
  if (stats) *stats = S0;
}

// ---------------------------------------------------------------------------
// Direct block-diffusion decoding (GravityOCR review, section 2 "Block
// Diffusion" and Appendix B.1; Trillion Labs blog, "confidence threshold").
// ---------------------------------------------------------------------------
struct DDOut {
  int steps, n, eos, advanced;
  int32_t tok[SSB_MAX_BLOCK];
  int32_t step_of[SSB_MAX_BLOCK];
};

// One block of B positions after the boundary of one request: denoising steps
// (draft-mode forward over [x0, s_1..s_B], then the commit rule on the device)
// until every position is committed, then, by write_mode, the cache-write
// forward: 1 always, 0 never, 2 unless the output ends in this block (EOS
// inside or max_commit <= B).  The host reads one small record per step.
void dd_block_impl(ssb_model* m, ssb_kv* kv, int B, float tau, int max_commit, int write_mode, float* step_conf,
                   int32_t* step_tok, float* step_logits, DDOut* out, hipStream_t st) {
  const ssb_config& c = m->c;
  check_model_kv(m, kv);
  if (kv->x0 < 0) fail(SSB_ESTATE, "direct diffusion needs a prefilled kv (no boundary token)");
  if (B < 1 || B > c.block_B) fail(SSB_EINVAL, "B must be in [1, block_B]");
  if (B + 1 > c.max_rows) fail(SSB_EINVAL, "B + 1 exceeds max_rows");
  if (tau != tau) fail(SSB_EINVAL, "tau must not be NaN");
  if (max_commit < 1) fail(SSB_EINVAL, "max_commit must be >= 1");
  if (write_mode < 0 || write_mode > 2) fail(SSB_EINVAL, "bad cache-write mode");
  if (kv->seq_len + B + 1 > c.max_positions) fail(SSB_ENOKV, "window exceeds max_positions");
  kv_ensure(kv, kv->seq_len + B + 1, st);
  ssb_pool* pool = kv->pool;
  ReqArgs ra = single_req(kv, B, max_commit);
  ra.win[0] = m->dd_win;
  ra.tau = tau;
  upload_req(m, ra, st);
  hip_check(launch_dd_init(m->req_dev, 1, c.mask_id, m->dd_rec, kDDRec, st), "direct diffusion init");
  const int p = kv->seq_len;
  auto step_body = [&](hipStream_t s, bool graph, float* logits) {
    FwdSpec f{};
    f.mode = PREP_DRAFT;
    f.M = B + 1;
    f.ra = ra;
    f.max_pos = p + B + 1;
    f.slots = slot_bucket(m, f.max_pos);
    f.graph = graph;
    f.logits = logits;
    f.stat_sc = kLog2e;
    run_forward(m, pool, f, s);
    hip_check(launch_dd_select(m->am_tok, m->am_z, m->req_dev, 1, c.mask_id, c.vocab, m->dd_rec, kDDRec, s),
              "direct diffusion select");
    hip_check(hipMemcpyAsync(m->pin_i32, m->dd_rec, (size_t)kDDRec * 4, hipMemcpyDeviceToHost, s),
              "copy step record");
  };
  const bool eager = step_logits || m->prof_kind >= 0;
  int steps = 0;
  const int32_t* o = m->pin_i32;
  for (;;) {
    if (eager) {
      step_body(st, false, step_logits ? step_logits + (size_t)steps * (B + 1) * c.vocab : nullptr);
    } else {
      hipGraphExec_t ex = get_graph(m, 2, pool, 1, B, slot_bucket(m, p + B + 1),
                                    [&](hipStream_t s) { step_body(s, true, nullptr); });
      hip_check(hipGraphLaunch(ex, st), "direct diffusion step graph launch");
    }
    hip_check(hipStreamSynchronize(st), "direct diffusion step sync");
    prof_collect(m);
    if (o[2]) fail(SSB_EHIP, "direct diffusion step produced an invalid token or confidence (NaN logits?)");
    if (o[0] < 1 || o[3] != steps + 1 || o[1] < 0 || o[1] >= B)
      fail(SSB_EHIP, "direct diffusion step record is inconsistent");
    for (int j = 0; j < B; ++j) {
      if (step_conf) std::memcpy(step_conf + (size_t)steps * B + j, o + 4 + 2 * B + j, 4);
      if (step_tok) step_tok[(size_t)steps * B + j] = o[4 + 3 * B + j];
    }
    ++steps;
    if (o[1] == 0) break;
    if (steps >= B) fail(SSB_EHIP, "direct diffusion block not complete after B steps");
  }
  out->steps = steps;
  out->eos = 0;
  out->n = B;
  for (int j = 0; j < B; ++j) {
    out->tok[j] = o[4 + B + j];
    out->step_of[j] = o[4 + j];
    if (out->tok[j] < 0 || out->tok[j] >= c.vocab || out->tok[j] == c.mask_id)
      fail(SSB_EHIP, "direct diffusion block holds an invalid token");
  }
  for (int j = 0; j < B; ++j)
    if (out->tok[j] == c.eos_id) { out->n = j + 1; out->eos = 1; break; }
  out->n = std::min(out->n, max_commit);
  const bool write = write_mode == 1 || (write_mode == 2 && !out->eos && max_commit > B);
  out->advanced = write ? 1 : 0;
  if (write) {
    if (B > 1) {
      // causal forward over s_1..s_{B-1} at p+1..p+B-1: a verify-mode window of B-1 rows
      ReqArgs rc = ra;
      rc.B = B - 2;
      upload_req(m, rc, st);    // the stream is idle: the staging buffer is free
      auto cw_body = [&](hipStream_t s, bool graph) {
        FwdSpec f{};
        f.mode = PREP_VERIFY;
        f.M = B - 1;
        f.ra = rc;
        f.max_pos = p + B;
        f.slots = slot_bucket(m, f.max_pos);
        f.graph = graph;
        f.no_head = true;
        run_forward(m, pool, f, s);
      };
      if (eager) {
        cw_body(st, false);
      } else {
        hipGraphExec_t ex = get_graph(m, 3, pool, 1, B, slot_bucket(m, p + B), [&](hipStream_t s) { cw_body(s, true); });
        hip_check(hipGraphLaunch(ex, st), "cache-write graph launch");
      }
      hip_check(hipStreamSynchronize(st), "cache-write sync");
      prof_collect(m);
    }
    kv->seq_len = p + B;
    kv->x0 = out->tok[B - 1];
  }
  kv_trim(kv, kv->seq_len + B + 1);
}

// Self-speculative round whose draft is refined by up to `steps` denoising
// steps (Trillion Labs blog, the draft-schedule passage; GravityOCR review,
// Appendix D): the direct-diffusion step kernels fill the window slots by the
// draft-side threshold, the last step commits the rest, then the greedy verify
// and accept of ssb_round run on [a0, d_1..d_B] read from the slots.
void round_multistep_impl(ssb_model* m, ssb_kv* kv, int B, int steps, float tau, int max_commit, float* vlog,
                          RoundOut* out, int* draft_forwards, hipStream_t st) {
  const ssb_config& c = m->c;
  check_model_kv(m, kv);
  if (kv->x0 < 0) fail(SSB_ESTATE, "round needs a prefilled kv (no boundary token)");
  if (B < 1 || B > c.block_B) fail(SSB_EINVAL, "B must be in [1, block_B]");
  if (B + 1 > c.max_rows) fail(SSB_EINVAL, "B + 1 exceeds max_rows");
  if (steps < 1) fail(SSB_EINVAL, "steps must be >= 1");
  if (tau != tau) fail(SSB_EINVAL, "tau must not be NaN");
  if (max_commit < 1) fail(SSB_EINVAL, "max_commit must be >= 1");
  if (kv->seq_len + B + 2 > c.max_positions) fail(SSB_ENOKV, "window exceeds max_positions");
  kv_ensure(kv, kv->seq_len + B + 2, st);
  ssb_pool* pool = kv->pool;
  ReqArgs ra = single_req(kv, B, max_commit);
  ra.win[0] = m->dd_win;
  ra.tau = tau;
  ra.dsteps = steps;
  upload_req(m, ra, st);
  hip_check(launch_dd_init(m->req_dev, 1, c.mask_id, m->dd_rec, kDDRec, st), "draft schedule init");
  const int p = kv->seq_len;
  const bool eager = vlog || m->prof_kind >= 0;
  auto step_body = [&](hipStream_t s, bool graph) {
    FwdSpec f{};
    f.mode = PREP_DRAFT;
    f.M = B + 1;
    f.ra = ra;
    f.max_pos = p + B + 1;
    f.slots = slot_bucket(m, f.max_pos);
    f.graph = graph;
    f.stat_sc = kLog2e;
    run_forward(m, pool, f, s);
    hip_check(launch_dd_select(m->am_tok, m->am_z, m->req_dev, 1, c.mask_id, c.vocab, m->dd_rec, kDDRec, s),
              "draft schedule select");
    hip_check(hipMemcpyAsync(m->pin_i32, m->dd_rec, (size_t)kDDRec * 4, hipMemcpyDeviceToHost, s),
              "copy step record");
  };
  int k = 0;
  for (;;) {
    if (eager) {
      step_body(st, false);
    } else {
      hipGraphExec_t ex = get_graph(m, 2, pool, 1, B, slot_bucket(m, p + B + 1),
                                    [&](hipStream_t s) { step_body(s, true); });
      hip_check(hipGraphLaunch(ex, st), "draft step graph launch");
    }
    hip_check(hipStreamSynchronize(st), "draft step sync");
    prof_collect(m);
    const int32_t* o = m->pin_i32;
    if (o[2]) fail(SSB_EHIP, "draft step produced an invalid token or confidence (NaN logits?)");
    if (o[0] < 1 || o[3] != k + 1 || o[1] < 0 || o[1] >= B) fail(SSB_EHIP, "draft step record is inconsistent");
    ++k;
    if (o[1] == 0) break;
    if (k >= steps) fail(SSB_EHIP, "draft schedule incomplete after its last step");
  }
  *draft_forwards = k;
  auto verify_body = [&](hipStream_t s, bool graph) {
    FwdSpec f{};
    f.mode = PREP_VERIFY;
    f.M = B + 1;
    f.ra = ra;
    f.max_pos = p + B + 2;
    f.slots = slot_bucket(m, f.max_pos);
    f.graph = graph;
    f.logits = vlog;
    run_forward(m, pool, f, s);
    ProfStamp* ast = prof_begin(m, kKindAccept, s);
    hip_check(launch_accept(m->row_tok, m->am_tok, m->req_dev, 1, c.eos_id, m->accept_dev, kOutStride, s,
                            m->tail_err, ast), "accept");
    prof_end(m, kKindAccept, s);
    hip_check(hipMemcpyAsync(m->pin_i32, m->accept_dev, (size_t)kOutStride * 4, hipMemcpyDeviceToHost, s),
              "copy accept");
  };
  if (eager) {
    verify_body(st, false);
  } else {
    hipGraphExec_t ex = get_graph(m, 6, pool, 1, B, slot_bucket(m, p + B + 2),
                                  [&](hipStream_t s) { verify_body(s, true); });
    hip_check(hipGraphLaunch(ex, st), "verify graph launch");
  }
  hip_check(hipStreamSynchronize(st), "verify sync");
  prof_collect(m);
  read_accept(m->pin_i32, B, c.vocab, c.mask_id, out);
  commit_round(*kv, *kv, *kv->pool, p, *out, B);
}


}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free rounds (ssb_round_noalloc): the forward workspace of one window laid out in a
// file-scope device array instead of the model's workspace.  Every GPU the library runs on holds
// its own copy of the array until the process ends; calls on one GPU share it.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)16 << 20;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kScratchDevices] = {};   // device address of each device's scratch array

// Once per device, with that device current (from ssb_init_model): the array's device address.
void scratch_setup(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return;   // ssb_round_noalloc then reports SSB_ESTATE
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return;
  void* ptr = nullptr;
  hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch symbol address");
  g_scratch[dev] = ptr;
}

// The workspace of one decode window of M rows (one request) whose attention reaches `chunks` key
// chunks, laid out from base (null: sizes only).  Returns the bytes it spans.  Every buffer is
// written before it is read within a round, so nothing needs clearing between calls.
size_t scratch_layout(const ssb_model* m, int M, int chunks, char* base, Workspace* ws) {
  const ssb_config& c = m->c;
  const size_t H = c.hidden, qd = (size_t)c.n_heads * c.head_dim, hd = c.head_dim, E = m->elem;
  const size_t n_groups = m->lm.n_tiles / m->lm.NT;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return base ? base + o : nullptr;
  };
  ws->h = reinterpret_cast<float*>(take(M * H * 4));
  ws->xg = take(M * H * E);
  ws->ssq = reinterpret_cast<float*>(take(H / 16 * M * 4));
  ws->q = take(M * qd * E);
  ws->attn = take(M * qd * E);
  ws->act = take(M * (size_t)c.ffn * E);
  int32_t* meta = reinterpret_cast<int32_t*>(take(5 * (size_t)M * 4));
  ws->row_tok = meta;
  ws->row_pos = meta ? meta + M : nullptr;
  ws->row_lim = meta ? meta + 2 * M : nullptr;
  ws->row_req = meta ? meta + 3 * M : nullptr;
  ws->row_slot = meta ? meta + 4 * M : nullptr;
  ws->row_cs = reinterpret_cast<float2*>(take(M * (hd / 2) * sizeof(float2)));
  ws->pt_ld = chunks * (kKeyChunk / kPage);
  ws->fwd_pt = reinterpret_cast<int32_t*>(take((size_t)ws->pt_ld * 4));   // one request
  ws->part = reinterpret_cast<float*>(take(m->d[0].S > 1 ? (size_t)m->d[0].S * M * H * 4 : 0));
  float* am = reinterpret_cast<float*>(take(3 * (size_t)M * 4));
  ws->am_tok = reinterpret_cast<int32_t*>(am);
  ws->am_top1 = am ? am + M : nullptr;
  ws->am_top2 = am ? am + 2 * M : nullptr;
  float* amp = reinterpret_cast<float*>(take(n_groups * M * 12));
  ws->amv1 = amp;
  ws->amv2 = amp ? amp + n_groups * M : nullptr;
  ws->ami1 = amp ? reinterpret_cast<int32_t*>(amp + 2 * n_groups * M) : nullptr;
  ws->ams = nullptr;        // softmax sums: direct diffusion and sampling only
  ws->am_z = reinterpret_cast<float*>(take((size_t)M * 4));
  ws->slog_d = ws->slog_v = nullptr;
  float* sst = reinterpret_cast<float*>(take(4 * (size_t)M * 4));
  ws->smax_d = sst;
  ws->sz_d = sst ? sst + M : nullptr;
  ws->smax_v = sst ? sst + 2 * M : nullptr;
  ws->sz_v = sst ? sst + 3 * M : nullptr;
  ws->dd_win = ws->dd_rec = nullptr;
  ws->max_chunks = chunks;
  ws->apart = reinterpret_cast<float*>(take((size_t)M * c.n_heads * chunks * (hd + 4) * 4));
  ws->max_decode_rows = M;
  ws->accept_dev = reinterpret_cast<int32_t*>(take((size_t)kOutStride * 4));
  ws->tok_dev = reinterpret_cast<int32_t*>(take((size_t)M * 4));
  ws->req_dev = reinterpret_cast<ReqArgs*>(take(sizeof(ReqArgs)));
  return off;
}
}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* ssb_last_error(void) { return g_err.c_str(); }

int ssb_check_config(const ssb_config* cfg) {
  return guard([&] { check_config(cfg); });
}

int ssb_init_model(const ssb_config* cfg, const ssb_weights* w, void* stream, ssb_model** out) {
  return guard([&] { init_model(cfg, w, S(stream), out); });
}

void ssb_free_model(ssb_model* m) {
  if (!m) return;
  (void)hipSetDevice(m->device);
  (void)hipDeviceSynchronize();
  (void)hipFree(m->wmem);
  (void)hipFree(m->ws);
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  for (hipEvent_t e : m->prof_ev) (void)hipEventDestroy(e);
  if (m->prof_stamps) (void)hipFree(m->prof_stamps);
  (void)hipStreamDestroy(m->cap);
  (void)hipHostFree(m->req_pin);
  (void)hipHostFree(m->pin_i32);
  (void)hipHostFree(m->pin_f32);
  delete m;
}

int ssb_model_memory(const ssb_model* m, size_t* weight_bytes, size_t* workspace_bytes) {
  return guard([&] {
    if (!m) fail(SSB_EINVAL, "null model");
    if (weight_bytes) *weight_bytes = m->wmem_bytes;
    if (workspace_bytes) *workspace_bytes = m->ws_bytes;
  });
}

int ssb_pool_bytes(const ssb_model* m, int n_pages, size_t* bytes) {
  return guard([&] {
    if (!m || !bytes) fail(SSB_EINVAL, "null argument");
    if (n_pages < 1) fail(SSB_EINVAL, "n_pages must be >= 1");
    const ssb_config& c = m->c;
    *bytes = (size_t)c.n_layers * n_pages * 2 * c.n_kv_heads * kPage * c.head_dim * m->elem;
  });
}

int ssb_pool_init(ssb_model* m, void* dev_buf, size_t bytes, int n_pages, ssb_pool** out) {
  return guard([&] {
    if (!m || !dev_buf || !out) fail(SSB_EINVAL, "null argument");
    size_t need = 0;
    if (ssb_pool_bytes(m, n_pages, &need) != SSB_OK) fail(SSB_EINVAL, g_err);
    if (bytes < need) fail(SSB_EINVAL, "pool buffer smaller than ssb_pool_bytes");
    if (reinterpret_cast<uintptr_t>(dev_buf) % 256) fail(SSB_EINVAL, "pool buffer must be 256-byte aligned");
    auto* p = new ssb_pool();
    std::unique_ptr<ssb_pool> hold(p);
    p->m = m;
    p->base = static_cast<char*>(dev_buf);
    p->init(n_pages);
    *out = hold.release();
  });
}

void ssb_pool_free(ssb_pool* p) {
  if (!p) return;
  // Captured graphs bake in this pool's device buffer: drop them, so that a pool created later
  // at the same host address can never replay them.
  ssb_model* m = p->m;
  (void)hipSetDevice(m->device);
  (void)hipDeviceSynchronize();
  for (auto it = m->graphs.begin(); it != m->graphs.end();) {
    if (std::get<1>(it->first) == static_cast<void*>(p)) {
      m->graph_prof_kinds.erase(it->second);
      (void)hipGraphExecDestroy(it->second);
      it = m->graphs.erase(it);
    } else {
      ++it;
    }
  }
  delete p;
}

int ssb_pool_free_pages(const ssb_pool* p, int* n_free) {
  return guard([&] {
    if (!p || !n_free) fail(SSB_EINVAL, "null argument");
    *n_free = p->n_free();
  });
}

int ssb_kv_create(ssb_pool* p, int max_tokens, ssb_kv** out) {
  return guard([&] {
    if (!p || !out) fail(SSB_EINVAL, "null argument");
    *out = kv_new(p, max_tokens);
  });
}

void ssb_kv_free(ssb_kv* kv) { kv_delete(kv); }

int ssb_kv_reset(ssb_kv* kv) {
  return guard([&] {
    if (!kv) fail(SSB_EINVAL, "null kv");
    kv_trim(kv, 0);
    kv->seq_len = 0;
    kv->x0 = -1;
  });
}

int ssb_kv_rewind(ssb_kv* kv, int n, int32_t x0) {
  return guard([&] {
    if (!kv) fail(SSB_EINVAL, "null kv");
    check_rewind(*kv, n, x0, kv->pool->m->c.vocab, kv->pool->m->c.mask_id);
    kv->seq_len = n;
    kv->x0 = x0;
    kv_trim(kv, n + kv->pool->m->c.block_B + 2);
  });
}

int ssb_kv_state(const ssb_kv* kv, int* seq_len, int32_t* x0, int* pages_held) {
  return guard([&] {
    if (!kv) fail(SSB_EINVAL, "null kv");
    if (seq_len) *seq_len = kv->seq_len;
    if (x0) *x0 = kv->x0;
    if (pages_held) *pages_held = (int)kv->pages.size();
  });
}

int ssb_prefill(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int32_t* first_token, void* stream) {
  return guard([&] { prefill(m, kv, prefix_dev, P, first_token, S(stream)); });
}

int ssb_round(ssb_model* m, ssb_kv* kv, int B, int max_commit, const int32_t* planted_dev, int32_t* committed,
              int32_t* n_committed, int32_t* accept_len, float* draft_logits_dev, float* verify_logits_dev,
              void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    RoundOut ro{};
    ssb_kv* kvs[1] = {kv};
    int mc[1] = {max_commit};
    round_impl(m, kvs, 1, B, mc, planted_dev, nullptr, nullptr, nullptr, nullptr, draft_logits_dev,
               verify_logits_dev, &ro, S(stream));
    if (committed) std::memcpy(committed, ro.tok, (size_t)ro.n * 4);
    if (n_committed) *n_committed = ro.n;
    if (accept_len) *accept_len = ro.A;
  });
}

int ssb_round_noalloc(ssb_model* m, ssb_kv* kv, int B, int max_commit, const int32_t* planted_dev,
                      int32_t* committed, int32_t* n_committed, int32_t* accept_len, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (B < 0 || B > m->c.block_B) fail(SSB_EINVAL, "B must be in [0, block_B]");
    char* base = m->device >= 0 && m->device < kScratchDevices ? static_cast<char*>(g_scratch[m->device]) : nullptr;
    if (!base) fail(SSB_ESTATE, "no scratch array address for this device");
    const int M = B + 1;
    const int chunks = (kv->seq_len + B + 2 - 1) / kKeyChunk + 1;   // keys of the verify window's last row
    Workspace ws{};
    const size_t need = scratch_layout(m, M, chunks, nullptr, &ws);
    if (need > kScratchBytes)
      fail(SSB_EINVAL, "ssb_round_noalloc: a window of " + std::to_string(M) + " rows over " +
                           std::to_string(kv->seq_len + B + 2) + " positions needs " + std::to_string(need) +
                           " bytes of scratch; the maximum is " + std::to_string(kScratchBytes));
    scratch_layout(m, M, chunks, base, &ws);
    // the model's workspace pointers name the scratch layout for this call only; launches run
    // eagerly (a captured graph would hold the other layout, and instantiating one allocates)
    struct Restore {
      ssb_model* m;
      Workspace w;
      bool no_graph;
      ~Restore() {
        static_cast<Workspace&>(*m) = w;
        m->no_graph = no_graph;
      }
    } restore{m, static_cast<const Workspace&>(*m), m->no_graph};
    static_cast<Workspace&>(*m) = ws;
    m->no_graph = true;
    RoundOut ro{};
    ssb_kv* kvs[1] = {kv};
    int mc[1] = {max_commit};
    round_impl(m, kvs, 1, B, mc, planted_dev, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &ro, S(stream));
    if (committed) std::memcpy(committed, ro.tok, (size_t)ro.n * 4);
    if (n_committed) *n_committed = ro.n;
    if (accept_len) *accept_len = ro.A;
  });
}

int ssb_ar_step(ssb_model* m, ssb_kv* kv, int32_t* token, float* logits_dev, void* stream) {
  return guard([&] { ar_step(m, kv, token, logits_dev, S(stream)); });
}

int ssb_decode(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, int max_len, const int32_t* cont_dev,
               int cont_len, const int32_t* astar, int n_astar, int32_t* out, int32_t* n_out, ssb_stats* stats,
               void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    if (B < 0 || B > m->c.block_B) fail(SSB_EINVAL, "B must be in [0, block_B]");
    if (cont_dev && cont_len < 0) fail(SSB_EINVAL, "negative cont_len");
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y1 = 0;
      prefill(m, kv, prefix_dev, P, &y1, S(stream));
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y1;
      bool done = y1 == m->c.eos_id || n >= max_len;
      int k = 0;
      while (!done) {
        RoundOut ro{};
        ssb_kv* kvs[1] = {kv};
        int mc[1] = {max_len - n};
        const bool plant = cont_dev && astar && k < n_astar;
        const int32_t* conts[1] = {cont_dev};
        int cl[1] = {cont_len}, cc[1] = {n}, as[1] = {plant ? astar[k] : 0};
        round_impl(m, kvs, 1, B, mc, nullptr, plant ? conts : nullptr, plant ? cl : nullptr, plant ? cc : nullptr,
                   plant ? as : nullptr, nullptr, nullptr, &ro, S(stream));
        for (int i = 0; i < ro.n; ++i) out[n++] = ro.tok[i];
        st.rounds += 1;
        st.forwards += 2;
        st.accepted += ro.A;
        done = ro.eos || n >= max_len;
        ++k;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_decode_ar(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int max_len, int32_t* out, int32_t* n_out,
                  ssb_stats* stats, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y = 0;
      prefill(m, kv, prefix_dev, P, &y, S(stream));
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y;
      while (y != m->c.eos_id && n < max_len) {
        ar_step(m, kv, &y, nullptr, S(stream));
        out[n++] = y;
        st.rounds += 1;
        st.forwards += 1;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_round_batch(ssb_model* m, ssb_kv* const* kvs, int R, int B, const int32_t* max_commit,
                    const int32_t* planted_dev, int32_t* committed, int32_t* n_committed, int32_t* accept_len,
                    float* draft_logits_dev, float* verify_logits_dev, void* stream) {
  return guard([&] {
    if (!m || !kvs || !max_commit) fail(SSB_EINVAL, "null argument");
    if (R < 1 || R > m->max_batch) fail(SSB_EINVAL, "R must be in [1, max_batch]");
    for (int r = 0; r < R; ++r)
      if (!kvs[r]) fail(SSB_EINVAL, "null kv in batch");
    std::vector<RoundOut> ro(R);
    std::vector<int> mc(max_commit, max_commit + R);
    round_impl(m, kvs, R, B, mc.data(), planted_dev, nullptr, nullptr, nullptr, nullptr, draft_logits_dev,
               verify_logits_dev, ro.data(), S(stream));
    for (int r = 0; r < R; ++r) {
      if (committed) std::memcpy(committed + (size_t)r * (B + 2), ro[r].tok, (size_t)ro[r].n * 4);
      if (n_committed) n_committed[r] = ro[r].n;
      if (accept_len) accept_len[r] = ro[r].A;
    }
  });
}

int ssb_kv_poison(ssb_kv* kv, int lo, int hi, void* stream) {
  return guard([&] {
    if (!kv) fail(SSB_EINVAL, "null kv");
    if (lo < 0 || hi < lo || hi > (int)kv->pages.size() * kPage) fail(SSB_EINVAL, "range outside the kv's pages");
    if (hi == lo) return;
    ssb_model* m = kv->pool->m;
    hipStream_t st = S(stream);
    ReqArgs ra = single_req(kv, 0, 1);
    upload_req(m, ra, st);
    poison_kv(m, kv->pool, 1, nullptr, st, lo, hi);
    hip_check(hipStreamSynchronize(st), "poison sync");
  });
}

int ssb_set_debug(ssb_model* m, int flags) {
  return guard([&] {
    if (!m) fail(SSB_EINVAL, "null model");
    if (flags & ~(SSB_DEBUG_POISON | SSB_DEBUG_UNFUSED)) fail(SSB_EINVAL, "unknown debug flag");
    m->debug_poison = (flags & SSB_DEBUG_POISON) != 0;
    const bool no_fused = (flags & SSB_DEBUG_UNFUSED) != 0;
    if (no_fused != m->no_fused) {
      // captured graphs hold the other form of the layer tail
      hip_check(hipDeviceSynchronize(), "sync before dropping graphs");
      for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
      m->graphs.clear();
      m->graph_prof_kinds.clear();
      m->no_fused = no_fused;
    }
  });
}

int ssb_round_sample(ssb_model* m, ssb_kv* kv, int B, int max_commit, float temperature, const float* u_dev,
                     int32_t* committed, int32_t* n_committed, int32_t* accept_len, float* draft_logits_dev,
                     float* verify_logits_dev, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    RoundOut ro{};
    ssb_kv* kvs[1] = {kv};
    int mc[1] = {max_commit};
    const float* us[1] = {u_dev};
    const SampleSpec smp{temperature, us};
    round_impl(m, kvs, 1, B, mc, nullptr, nullptr, nullptr, nullptr, nullptr, draft_logits_dev, verify_logits_dev,
               &ro, S(stream), &smp);
    if (committed) std::memcpy(committed, ro.tok, (size_t)ro.n * 4);
    if (n_committed) *n_committed = ro.n;
    if (accept_len) *accept_len = ro.A;
  });
}

int ssb_decode_sample(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, float temperature,
                      int max_len, const float* u_dev, int n_u_rows, int32_t* out, int32_t* n_out, ssb_stats* stats,
                      void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    if (B < 0 || B > m->c.block_B) fail(SSB_EINVAL, "B must be in [0, block_B]");
    if (!u_dev || n_u_rows < 1) fail(SSB_EINVAL, "null uniforms");
    const int W = 2 * B + 2;
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y1 = 0;
      const float* u0[1] = {u_dev};
      const SampleSpec s0{temperature, u0};
      prefill(m, kv, prefix_dev, P, &y1, S(stream), &s0);
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y1;
      bool done = y1 == m->c.eos_id || n >= max_len;
      int k = 1;
      while (!done) {
        if (k >= n_u_rows) fail(SSB_EINVAL, "more rounds than rows of uniforms");
        RoundOut ro{};
        ssb_kv* kvs[1] = {kv};
        int mc[1] = {max_len - n};
        const float* us[1] = {u_dev + (size_t)k * W};
        const SampleSpec smp{temperature, us};
        round_impl(m, kvs, 1, B, mc, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &ro, S(stream),
                   &smp);
        for (int i = 0; i < ro.n; ++i) out[n++] = ro.tok[i];
        st.rounds += 1;
        st.forwards += 2;
        st.accepted += ro.A;
        done = ro.eos || n >= max_len;
        ++k;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_decode_ar_sample(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, float temperature, int max_len,
                         const float* u_dev, int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    if (!u_dev) fail(SSB_EINVAL, "null uniforms");
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y = 0;
      const float* u0[1] = {u_dev};
      const SampleSpec s0{temperature, u0};
      prefill(m, kv, prefix_dev, P, &y, S(stream), &s0);
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y;
      while (y != m->c.eos_id && n < max_len) {
        const float* uk[1] = {u_dev + n};
        const SampleSpec sk{temperature, uk};
        ar_step(m, kv, &y, nullptr, S(stream), &sk);
        out[n++] = y;
        st.rounds += 1;
        st.forwards += 1;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_round_multistep(ssb_model* m, ssb_kv* kv, int B, int steps, float tau, int max_commit, int32_t* committed,
                        int32_t* n_committed, int32_t* accept_len, int32_t* draft_forwards, float* verify_logits_dev,
                        void* stream) {
  return guard([&] {
    RoundOut ro{};
    int k = 0;
    round_multistep_impl(m, kv, B, steps, tau, max_commit, verify_logits_dev, &ro, &k, S(stream));
    if (committed) std::memcpy(committed, ro.tok, (size_t)ro.n * 4);
    if (n_committed) *n_committed = ro.n;
    if (accept_len) *accept_len = ro.A;
    if (draft_forwards) *draft_forwards = k;
  });
}

int ssb_decode_multistep(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, int steps, float tau,
                         int max_len, int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    if (B < 1 || B > m->c.block_B) fail(SSB_EINVAL, "B must be in [1, block_B]");
    if (steps < 1) fail(SSB_EINVAL, "steps must be >= 1");
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y1 = 0;
      prefill(m, kv, prefix_dev, P, &y1, S(stream));
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y1;
      bool done = y1 == m->c.eos_id || n >= max_len;
      while (!done) {
        RoundOut ro{};
        int k = 0;
        round_multistep_impl(m, kv, B, steps, tau, max_len - n, nullptr, &ro, &k, S(stream));
        for (int i = 0; i < ro.n; ++i) out[n++] = ro.tok[i];
        st.rounds += 1;
        st.forwards += k + 1;
        st.accepted += ro.A;
        done = ro.eos || n >= max_len;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_ar_step_batch(ssb_model* m, ssb_kv* const* kvs, int R, int32_t* tokens, void* stream) {
  return guard([&] {
    if (!m || !kvs || !tokens) fail(SSB_EINVAL, "null argument");
    if (R < 1 || R > m->max_batch) fail(SSB_EINVAL, "R must be in [1, max_batch]");
    for (int r = 0; r < R; ++r)
      if (!kvs[r]) fail(SSB_EINVAL, "null kv in batch");
    ar_step_batch_impl(m, kvs, R, tokens, S(stream));
  });
}

int ssb_serve(ssb_model* m, ssb_pool* pool, ssb_request* reqs, int n_reqs, int max_running, int mode, int B,
              int max_tokens, ssb_serve_stats* stats, void* stream) {
  return guard([&] {
    if (!m || !pool) fail(SSB_EINVAL, "null argument");
    hip_check(hipSetDevice(m->device), "hipSetDevice");
    serve_impl(m, pool, reqs, n_reqs, max_running, mode, B, max_tokens, stats, S(stream));
  });
}

int ssb_dd_block(ssb_model* m, ssb_kv* kv, int B, float tau, int max_commit, int write_cache, int32_t* tokens,
                 int32_t* n_tokens, int32_t* steps, int32_t* step_of, float* step_conf, int32_t* step_tok,
                 float* step_logits_dev, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (write_cache != 0 && write_cache != 1) fail(SSB_EINVAL, "write_cache must be 0 or 1");
    DDOut o{};
    dd_block_impl(m, kv, B, tau, max_commit, write_cache, step_conf, step_tok, step_logits_dev, &o, S(stream));
    if (tokens) std::memcpy(tokens, o.tok, (size_t)B * 4);
    if (step_of) std::memcpy(step_of, o.step_of, (size_t)B * 4);
    if (n_tokens) *n_tokens = o.n;
    if (steps) *steps = o.steps;
  });
}

int ssb_decode_dd(ssb_model* m, ssb_kv* kv, const void* prefix_dev, int P, int B, float tau, int max_len,
                  int32_t* out, int32_t* n_out, ssb_stats* stats, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (max_len < 0) fail(SSB_EINVAL, "max_len must be >= 0");
    if (max_len > 0 && !out) fail(SSB_EINVAL, "null output buffer");
    if (B < 1 || B > m->c.block_B) fail(SSB_EINVAL, "B must be in [1, block_B]");
    if (tau != tau) fail(SSB_EINVAL, "tau must not be NaN");
    ssb_stats st{};
    int n = 0;
    if (max_len > 0) {
      const double t0 = now_us();
      int32_t y1 = 0;
      prefill(m, kv, prefix_dev, P, &y1, S(stream));
      const double t1 = now_us();
      st.prefill_us = t1 - t0;
      out[n++] = y1;
      bool done = y1 == m->c.eos_id || n >= max_len;
      while (!done) {
        DDOut o{};
        dd_block_impl(m, kv, B, tau, max_len - n, 2, nullptr, nullptr, nullptr, &o, S(stream));
        for (int i = 0; i < o.n; ++i) out[n++] = o.tok[i];
        st.rounds += 1;
        st.forwards += o.steps;
        st.cache_forwards += (o.advanced && B > 1) ? 1 : 0;
        done = o.eos || n >= max_len;
      }
      st.decode_us = now_us() - t1;
    }
    st.tokens = n;
    if (n_out) *n_out = n;
    if (stats) *stats = st;
  });
}

int ssb_forward_tokens(ssb_model* m, ssb_kv* kv, const int32_t* tokens, int M, int p, float* logits_dev,
                       int32_t* argmax, float* top1, float* top2, void* stream) {
  return guard([&] {
    check_model_kv(m, kv);
    if (!tokens || !argmax) fail(SSB_EINVAL, "null tokens or argmax");
    if (M < 1 || M > m->c.max_rows) fail(SSB_EINVAL, "M must be in [1, max_rows]");
    if (p < 0 || p > kv->seq_len) fail(SSB_EINVAL, "p must be within the committed length");
    if (p + M > m->c.max_positions) fail(SSB_ENOKV, "positions exceed max_positions");
    for (int i = 0; i < M; ++i)
      if (tokens[i] < 0 || tokens[i] >= m->c.vocab) fail(SSB_EINVAL, "token id out of range");
    hipStream_t st = S(stream);
    kv_ensure(kv, p + M, st);
    std::memcpy(m->pin_i32, tokens, (size_t)M * 4);
    hip_check(hipMemcpyAsync(m->tok_dev, m->pin_i32, (size_t)M * 4, hipMemcpyHostToDevice, st), "upload tokens");
    FwdSpec f{};
    f.mode = PREP_TOKENS;
    f.M = M;
    f.pos0 = p;
    f.ra = single_req(kv, 0, 1);
    upload_req(m, f.ra, st);
    f.max_pos = p + M;
    f.logits = logits_dev;
    run_forward(m, kv->pool, f, st);
    hip_check(hipStreamSynchronize(st), "sync before reuse of staging");
    hip_check(hipMemcpyAsync(m->pin_i32, m->am_tok, (size_t)M * 4, hipMemcpyDeviceToHost, st), "copy argmax");
    hip_check(hipMemcpyAsync(m->pin_f32, m->am_top1, (size_t)M * 4, hipMemcpyDeviceToHost, st), "copy top1");
    hip_check(hipMemcpyAsync(m->pin_f32 + m->c.max_rows, m->am_top2, (size_t)M * 4, hipMemcpyDeviceToHost, st),
              "copy top2");
    hip_check(hipStreamSynchronize(st), "forward sync");
    prof_collect(m);
    std::memcpy(argmax, m->pin_i32, (size_t)M * 4);
    if (top1) std::memcpy(top1, m->pin_f32, (size_t)M * 4);
    if (top2) std::memcpy(top2, m->pin_f32 + m->c.max_rows, (size_t)M * 4);
    // positions beyond the committed length hold no committed state
    kv_trim(kv, std::max(kv->seq_len + m->c.block_B + 2, 0));
  });
}

int ssb_profile_kernel(ssb_model* m, int kind) {
  return guard([&] {
    if (!m) fail(SSB_EINVAL, "null model");
    const bool in_graph = kind >= 0 && (kind & SSB_PROFILE_IN_GRAPH);
    if (kind >= 0) kind &= ~SSB_PROFILE_IN_GRAPH;
    if (kind < -1 || kind > SSB_K_TAIL) fail(SSB_EINVAL, "unknown kernel kind");
    hip_check(hipSetDevice(m->device), "hipSetDevice");
    if (kind >= 0 && m->prof_ev.empty()) {
      // two forwards of a round launch each kind at most n_layers + 1 times, plus prefill chunks
      const int pairs = 8 * (m->c.n_layers + 2);
      m->prof_ev.resize(2 * pairs);
      for (auto& e : m->prof_ev) hip_check(hipEventCreate(&e), "event create");
    }
    if (in_graph && !m->prof_stamps) {
      m->prof_slots = 32 * (m->c.n_layers + 2);   // every launch of a graph has a slot
      hip_check(hipMalloc(reinterpret_cast<void**>(&m->prof_stamps), m->prof_slots * sizeof(ProfStamp)),
                "stamp slots");
      hip_check(hipMemset(m->prof_stamps, 0, m->prof_slots * sizeof(ProfStamp)), "clear stamps");
      int khz = 0;
      hip_check(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, m->device), "wall clock rate");
      if (khz > 0) m->wallclock_mhz = khz / 1000.0;
    }
    m->prof_kind = kind;
    m->prof_graph = in_graph;
    m->prof_used = 0;
    m->prof_stamp_used = 0;
  });
}

int ssb_profile_read(ssb_model* m, double* total_us, long long* launches, int reset) {
  return guard([&] {
    if (!m) fail(SSB_EINVAL, "null model");
    if (total_us) *total_us = m->prof_us;
    if (launches) *launches = m->prof_launches;
    if (reset) { m->prof_us = 0; m->prof_launches = 0; }
  });
}

}  // extern "C"
