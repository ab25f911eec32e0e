// Host-side bookkeeping of the round engine, free of GPU calls so that it also builds as a plain
// CPU program (a sanitizer-instrumented check exercises it on its own): the configuration check,
// the KV page allocator, the sequence state that a round commits and rolls back (GravityOCR review,
// section 3.2 and Appendix B.2: after a round the cache holds x0, a0, d_1..d_A at p..p+A+1 and the
// new boundary is a_{A+1}), the accept record, and the conversion of errors into ABI codes.
#pragma once
#include <stdint.h>

#include <new>
#include <string>
#include <vector>

#include "../../include/ssb.h"
#include "ssb_limits.h"

namespace ssb {

struct Error {
  int code;
  std::string msg;
};

[[noreturn]] inline void fail(int code, const std::string& msg) { throw Error{code, msg}; }

// Runs f; what it throws becomes an ABI code with its message in *msg (SSB_OK if nothing is).
template <typename F>
int run_guarded(F&& f, std::string* msg) {
  try {
    f();
    return SSB_OK;
  } catch (const Error& e) {
    *msg = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    *msg = "host allocation failed";
    return SSB_ENOMEM;
  } catch (...) {
    *msg = "unexpected internal error";
    return SSB_EINVAL;
  }
}

inline bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Pages that hold positions [0, tokens) (none for tokens <= 0), with no overflow near INT_MAX.
inline int pages_for(int tokens) { return tokens <= 0 ? 0 : tokens / kPage + (tokens % kPage != 0); }

// The shapes and ids the kernels support; SSB_EINVAL with the first violated rule otherwise.
inline void check_config(const ssb_config* c) {
  if (!c) fail(SSB_EINVAL, "null config");
  auto req = [](bool ok, const char* m) {
    if (!ok) fail(SSB_EINVAL, m);
  };
  req(c->dtype == SSB_BF16 || c->dtype == SSB_F32, "dtype must be SSB_BF16 or SSB_F32");
  req(c->n_layers >= 1, "n_layers must be >= 1");
  req(c->head_dim == 32 || c->head_dim == 64, "head_dim must be 32 or 64");
  req(c->n_heads >= 1 && c->n_kv_heads >= 1 && c->n_heads % c->n_kv_heads == 0,
      "n_heads must be a multiple of n_kv_heads");
  req(c->n_heads / c->n_kv_heads == 1 || c->n_heads / c->n_kv_heads == 4, "n_heads/n_kv_heads must be 1 or 4");
  req(c->hidden % 128 == 0 && pow2(c->hidden / 128), "hidden must be 128 * 2^k");
  const long long qd = (long long)c->n_heads * c->head_dim;   // no int overflow for huge head counts
  req(qd <= (c->dtype == SSB_BF16 ? 4096 : 2048),
      "n_heads*head_dim above 4096 (bf16) / 2048 (f32) is not supported");
  req(qd % 128 == 0 && pow2((int)(qd / 128)), "n_heads*head_dim must be 128 * 2^k");
  req(c->ffn % 128 == 0 && pow2(c->ffn / 128), "ffn must be 128 * 2^k");
  req(c->hidden <= 16 * kMaxNormParts, "hidden above 2048 is not supported");
  req(c->hidden <= (c->dtype == SSB_BF16 ? 4096 : 2048),
      "hidden above 4096 (bf16) / 2048 (f32) is not supported");
  // the down projection (reduction length ffn) splits K over workgroups when one cannot hold it
  req(c->ffn <= (c->dtype == SSB_BF16 ? 8192 : 4096), "ffn above 8192 (bf16) / 4096 (f32) is not supported");
  req(c->vocab >= 2, "vocab must be >= 2");
  req(c->mask_id >= 0 && c->mask_id < c->vocab, "mask_id out of range");
  req(c->eos_id >= 0 && c->eos_id < c->vocab && c->eos_id != c->mask_id, "eos_id out of range or == mask_id");
  req(c->block_B >= 0 && c->block_B <= SSB_MAX_BLOCK, "block_B must be in [0, 64]");
  req(c->page_tokens == kPage, "page_tokens must be 16");
  req(c->max_rows >= 1 && c->max_rows <= kMaxTasks * kTaskRows, "max_rows must be in [1, 3072]");
  req(c->max_rows >= c->block_B + 1, "max_rows must hold one window (block_B + 1 rows)");
  req(c->max_positions >= 2, "max_positions must be >= 2");
  req(c->rms_eps >= 0.f && c->rope_theta > 0.f, "bad rms_eps or rope_theta");
  req(c->max_batch >= 0 && c->max_batch <= SSB_MAX_BATCH, "max_batch must be in [0, SSB_MAX_BATCH]");
  req((c->features & ~SSB_FEAT_SAMPLE) == 0, "unknown feature bits");
}

// The free pages of a pool: a stack of page ids, every id in [0, n_pages) at most once.
struct PageStack {
  int n_pages = 0;
  std::vector<int> free_pages;

  void init(int n) {
    if (n < 1) fail(SSB_EINVAL, "n_pages must be >= 1");
    n_pages = n;
    free_pages.clear();
    free_pages.reserve(n);
    for (int i = n - 1; i >= 0; --i) free_pages.push_back(i);
  }
  int n_free() const { return (int)free_pages.size(); }
};

// The pages one sequence holds, in logical order (logical page i covers positions 16i..16i+15),
// and the host mirror of its page table (max_pages entries, owned by the caller).
struct PageList {
  int max_tokens = 0;
  int max_pages = 0;
  std::vector<int32_t> pages;

  void init(int max_tok) {
    if (max_tok < 2) fail(SSB_EINVAL, "max_tokens must be >= 2");
    max_tokens = max_tok;
    max_pages = pages_for(max_tok);
    pages.clear();
    pages.reserve(max_pages);   // pushes on the round path never reallocate
  }

  // Holds pages for positions [0, n_tokens): takes the missing ones from the pool and writes their
  // ids into table[first..need).  Returns `first` (the page count before the call; no page was
  // added when it equals the count after).  SSB_ENOKV beyond max_tokens or when the pool has too
  // few free pages; nothing changes then.
  int ensure(PageStack& pool, int n_tokens, int32_t* table) {
    if (n_tokens > max_tokens) fail(SSB_ENOKV, "sequence would exceed the kv's max_tokens");
    const int need = pages_for(n_tokens);
    const int first = (int)pages.size();
    if (need <= first) return first;
    if (pool.n_free() < need - first) fail(SSB_ENOKV, "KV page pool exhausted");
    for (int i = first; i < need; ++i) {
      const int pg = pool.free_pages.back();
      pool.free_pages.pop_back();
      pages.push_back(pg);
      table[i] = pg;
    }
    return first;
  }

  // Returns to the pool every page wholly at positions >= keep_tokens (all of them for keep <= 0).
  void trim(PageStack& pool, int keep_tokens) {
    const int keep = pages_for(keep_tokens);
    while ((int)pages.size() > keep) {
      pool.free_pages.push_back(pages.back());
      pages.pop_back();
    }
  }
};

// What a sequence has committed: seq_len cached positions and the boundary token x0 at position
// seq_len, not yet cached (x0 = -1 before prefill).
struct SeqState {
  int seq_len = 0;
  int32_t x0 = -1;
};

// A rewind to n cached positions with boundary x0: n in [1, seq_len], x0 a token the model can emit.
inline void check_rewind(const SeqState& s, int n, int32_t x0, int vocab, int mask_id) {
  if (s.x0 < 0) fail(SSB_ESTATE, "rewind needs a prefilled kv");
  if (n < 1 || n > s.seq_len) fail(SSB_EINVAL, "n must be in [1, current length]");
  if (x0 < 0 || x0 >= vocab || x0 == mask_id) fail(SSB_EINVAL, "bad boundary token");
}

// Accept record of one request, written by the accept kernel:
// [A, n committed, next boundary a_{A+1}, EOS flag, committed tokens...].
constexpr int kOutStride = 4 + SSB_MAX_BLOCK + 2;

struct RoundOut {
  int A, n, next_x0, eos;
  int32_t tok[SSB_MAX_BLOCK + 2];
};

// Reads a record and checks what a correct round guarantees: 0 <= A <= B, 1 <= n <= A + 2 (fewer
// only at EOS or the commit budget), every committed token and the next boundary a real token.
// A record that breaks this (the kernels' answer to NaN logits) gives SSB_EHIP and *ro is unusable.
inline void read_accept(const int32_t* o, int B, int vocab, int mask_id, RoundOut* ro) {
  ro->A = o[0];
  ro->n = o[1];
  ro->next_x0 = o[2];
  ro->eos = o[3];
  auto tok_ok = [&](int32_t t) { return t >= 0 && t < vocab && t != mask_id; };
  if (ro->A < 0 || ro->A > B || ro->n < 1 || ro->n > ro->A + 2 || !tok_ok(ro->next_x0))
    fail(SSB_EHIP, "round produced an invalid accept record (NaN logits?)");
  for (int k = 0; k < ro->n; ++k) {
    ro->tok[k] = o[4 + k];
    if (!tok_ok(ro->tok[k])) fail(SSB_EHIP, "round produced an invalid committed token (NaN logits?)");
  }
}

// Commit and rollback of a round from boundary position p: the cache keeps x0, a0, d_1..d_A
// (length p + A + 2), the boundary becomes a_{A+1}, and pages past the next window's reach
// (p + A + 2 + B + 2 positions) go back to the pool.
inline void commit_round(SeqState& s, PageList& pl, PageStack& pool, int p, const RoundOut& ro, int B) {
  s.seq_len = p + ro.A + 2;
  s.x0 = ro.next_x0;
  pl.trim(pool, s.seq_len + B + 2);
}

// The end of a batched round of R requests (Seq: a PageList and a SeqState, e.g. a kv): every
// record (stride kOutStride) is read and checked before any request commits, so one bad record
// leaves every request's state as it was.
template <typename Seq>
void commit_batch(Seq* const* seqs, int R, PageStack& pool, const int* p, const int32_t* recs, int B, int vocab,
                  int mask_id, RoundOut* out) {
  for (int r = 0; r < R; ++r) read_accept(recs + (size_t)r * kOutStride, B, vocab, mask_id, &out[r]);
  for (int r = 0; r < R; ++r) commit_round(*seqs[r], *seqs[r], pool, p[r], out[r], B);
}

}  // namespace ssb
