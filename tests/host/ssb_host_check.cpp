// CPU check of the round engine's host bookkeeping (ssb_host.h), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py: the configuration check, the KV page
// allocator under a long random sequence of rounds, rewinds and resets on sequences that share a
// pool, the accept record, the transactional batch commit and the error conversion.
//
// Built with -DSSB_HOST_CHECK_CONTROL it instead hands PageList::ensure a page table one entry too
// short, so that a working AddressSanitizer build must stop it with a heap-buffer-overflow.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <random>
#include <set>
#include <vector>

#include "ssb_host.h"

using namespace ssb;

static int g_checks = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

// The code a call returns and whether its message contains `frag`.
template <typename F>
static int code_of(F&& f, const char* frag = nullptr) {
  std::string msg;
  const int rc = run_guarded(f, &msg);
  if (frag && rc != SSB_OK && msg.find(frag) == std::string::npos) {
    std::fprintf(stderr, "message '%s' lacks '%s'\n", msg.c_str(), frag);
    std::exit(1);
  }
  return rc;
}

static ssb_config base_config() {
  ssb_config c;
  std::memset(&c, 0, sizeof(c));
  c.dtype = SSB_BF16;
  c.n_layers = 24;
  c.hidden = 1024;
  c.n_heads = 16;
  c.n_kv_heads = 4;
  c.head_dim = 64;
  c.ffn = 4096;
  c.vocab = 60000;
  c.mask_id = 59999;
  c.eos_id = 59998;
  c.block_B = 32;
  c.page_tokens = 16;
  c.max_rows = 2048;
  c.max_positions = 5400;
  c.rms_eps = 1e-6f;
  c.rope_theta = 10000.f;
  c.max_batch = 1;
  c.features = 0;
  return c;
}

static void check_errors() {
  CHECK(code_of([] {}) == SSB_OK);
  CHECK(code_of([] { fail(SSB_ENOKV, "pool"); }, "pool") == SSB_ENOKV);
  CHECK(code_of([] { throw std::bad_alloc(); }, "allocation") == SSB_ENOMEM);
  CHECK(code_of([] { throw 7; }, "unexpected") == SSB_EINVAL);
}

static void check_configs() {
  ssb_config c = base_config();
  CHECK(code_of([&] { check_config(&c); }) == SSB_OK);
  CHECK(code_of([] { check_config(nullptr); }, "null") == SSB_EINVAL);
  struct Bad {
    void (*mutate)(ssb_config&);
    const char* frag;
  };
  const Bad bad[] = {
      {[](ssb_config& x) { x.dtype = 7; }, "dtype"},
      {[](ssb_config& x) { x.n_layers = 0; }, "n_layers"},
      {[](ssb_config& x) { x.head_dim = 128; }, "head_dim"},
      {[](ssb_config& x) { x.n_kv_heads = 3; }, "multiple"},
      {[](ssb_config& x) { x.n_kv_heads = 0; }, "multiple"},
      {[](ssb_config& x) { x.n_kv_heads = 8; }, "1 or 4"},
      {[](ssb_config& x) { x.hidden = 768; }, "hidden"},
      {[](ssb_config& x) { x.hidden = 4096; }, "2048"},
      {[](ssb_config& x) { x.ffn = 3072; }, "ffn"},
      {[](ssb_config& x) { x.ffn = 16384; }, "ffn"},
      {[](ssb_config& x) { x.vocab = 1; }, "vocab"},
      {[](ssb_config& x) { x.mask_id = 60000; }, "mask_id"},
      {[](ssb_config& x) { x.mask_id = -1; }, "mask_id"},
      {[](ssb_config& x) { x.eos_id = x.mask_id; }, "eos_id"},
      {[](ssb_config& x) { x.block_B = 65; }, "block_B"},
      {[](ssb_config& x) { x.block_B = -1; }, "block_B"},
      {[](ssb_config& x) { x.page_tokens = 32; }, "page_tokens"},
      {[](ssb_config& x) { x.max_rows = 0; }, "max_rows"},
      {[](ssb_config& x) { x.max_rows = 3073; }, "max_rows"},
      {[](ssb_config& x) { x.max_rows = 32; }, "one window"},
      {[](ssb_config& x) { x.max_positions = 1; }, "max_positions"},
      {[](ssb_config& x) { x.rms_eps = -1.f; }, "rms_eps"},
      {[](ssb_config& x) { x.rope_theta = 0.f; }, "rope_theta"},
      {[](ssb_config& x) { x.max_batch = 65; }, "max_batch"},
      {[](ssb_config& x) { x.max_batch = -1; }, "max_batch"},
      {[](ssb_config& x) { x.features = 2; }, "feature"},
      {[](ssb_config& x) { x.n_heads = INT_MAX; x.n_kv_heads = 1; }, "n_heads"},
      // n_heads * head_dim beyond INT_MAX must be refused, not wrapped
      {[](ssb_config& x) { x.n_heads = 1 << 26; x.n_kv_heads = 1 << 24; }, "n_heads*head_dim"},
  };
  for (const Bad& b : bad) {
    ssb_config x = base_config();
    b.mutate(x);
    CHECK(code_of([&] { check_config(&x); }, b.frag) == SSB_EINVAL);
  }
  ssb_config f = base_config();
  f.dtype = SSB_F32;
  f.hidden = 2048;
  f.n_heads = 32;
  f.n_kv_heads = 8;
  f.ffn = 4096;
  CHECK(code_of([&] { check_config(&f); }) == SSB_OK);
  f.ffn = 8192;
  CHECK(code_of([&] { check_config(&f); }, "ffn") == SSB_EINVAL);
  f = base_config();
  f.max_batch = 0;
  f.features = SSB_FEAT_SAMPLE;
  f.max_positions = INT_MAX;
  f.block_B = 0;
  f.max_rows = 1;
  CHECK(code_of([&] { check_config(&f); }) == SSB_OK);
}

static void check_pages_basic() {
  PageStack pool;
  CHECK(code_of([&] { pool.init(0); }, "n_pages") == SSB_EINVAL);
  pool.init(5);
  CHECK(pool.n_free() == 5);
  PageList pl;
  CHECK(code_of([&] { pl.init(1); }, "max_tokens") == SSB_EINVAL);
  pl.init(70);   // 5 pages
  CHECK(pl.max_pages == 5);
  std::unique_ptr<int32_t[]> table(new int32_t[pl.max_pages]);
  CHECK(pl.ensure(pool, 1, table.get()) == 0);
  CHECK(pl.pages.size() == 1 && pl.pages[0] == 0 && table[0] == 0);   // ids come out in order
  CHECK(pl.ensure(pool, 16, table.get()) == 1 && pl.pages.size() == 1);
  CHECK(pl.ensure(pool, 17, table.get()) == 1 && pl.pages.size() == 2 && table[1] == 1);
  CHECK(code_of([&] { pl.ensure(pool, 71, table.get()); }, "max_tokens") == SSB_ENOKV);
  CHECK(pl.pages.size() == 2 && pool.n_free() == 3);
  // a second sequence takes all but one free page; the first then cannot grow by two
  PageList other;
  other.init(64);
  std::unique_ptr<int32_t[]> t2(new int32_t[other.max_pages]);
  other.ensure(pool, 32, t2.get());
  CHECK(pool.n_free() == 1);
  CHECK(code_of([&] { pl.ensure(pool, 64, table.get()); }, "exhausted") == SSB_ENOKV);
  CHECK(pl.pages.size() == 2 && pool.n_free() == 1);                    // nothing moved
  CHECK(pl.ensure(pool, 48, table.get()) == 2 && pool.n_free() == 0);
  pl.trim(pool, 33);   // positions 0..32 need 3 pages
  CHECK(pl.pages.size() == 3);
  pl.trim(pool, 32);
  CHECK(pl.pages.size() == 2 && pool.n_free() == 1);
  pl.trim(pool, INT_MAX);   // no overflow, nothing freed
  CHECK(pl.pages.size() == 2);
  pl.trim(pool, -5);
  CHECK(pl.pages.empty() && pool.n_free() == 3);
  CHECK(pl.ensure(pool, -3, table.get()) == 0 && pl.pages.empty());
  CHECK(pages_for(INT_MAX) == INT_MAX / kPage + 1);
  CHECK(pages_for(0) == 0 && pages_for(1) == 1 && pages_for(16) == 1 && pages_for(17) == 2);
}

static void check_rewinds() {
  SeqState s;
  CHECK(code_of([&] { check_rewind(s, 1, 5, 100, 99); }, "prefilled") == SSB_ESTATE);
  s.seq_len = 40;
  s.x0 = 3;
  CHECK(code_of([&] { check_rewind(s, 1, 5, 100, 99); }) == SSB_OK);
  CHECK(code_of([&] { check_rewind(s, 40, 5, 100, 99); }) == SSB_OK);
  CHECK(code_of([&] { check_rewind(s, 0, 5, 100, 99); }, "current length") == SSB_EINVAL);
  CHECK(code_of([&] { check_rewind(s, 41, 5, 100, 99); }, "current length") == SSB_EINVAL);
  CHECK(code_of([&] { check_rewind(s, 10, 99, 100, 99); }, "boundary") == SSB_EINVAL);
  CHECK(code_of([&] { check_rewind(s, 10, 100, 100, 99); }, "boundary") == SSB_EINVAL);
  CHECK(code_of([&] { check_rewind(s, 10, -1, 100, 99); }, "boundary") == SSB_EINVAL);
}

// A record as the accept kernel writes it for A accepted drafts and n committed tokens.
static void make_record(int32_t* o, int A, int n, int next, int eos, int tok0) {
  o[0] = A;
  o[1] = n;
  o[2] = next;
  o[3] = eos;
  for (int k = 0; k < n; ++k) o[4 + k] = tok0 + k;
}

static void check_records() {
  const int B = 8, V = 100, MASK = 99;
  int32_t o[kOutStride];
  RoundOut ro;
  make_record(o, 3, 5, 40, 0, 10);
  CHECK(code_of([&] { read_accept(o, B, V, MASK, &ro); }) == SSB_OK);
  CHECK(ro.A == 3 && ro.n == 5 && ro.next_x0 == 40 && ro.tok[4] == 14);
  make_record(o, B, B + 2, 1, 0, 0);   // full accept commits B + 2
  CHECK(code_of([&] { read_accept(o, B, V, MASK, &ro); }) == SSB_OK);
  make_record(o, 0, 1, 1, 1, 0);       // EOS as a0
  CHECK(code_of([&] { read_accept(o, B, V, MASK, &ro); }) == SSB_OK);
  const int bad[][5] = {
      {-1, 1, 5, 0, 0},       // the kernels' mark of a failed launch
      {B + 1, 3, 5, 0, 0},    // more accepted than drafted
      {2, 0, 5, 0, 0},        // nothing committed
      {2, 5, 5, 0, 0},        // more than A + 2 committed
      {2, 3, MASK, 0, 0},     // [M] as the next boundary
      {2, 3, V, 0, 0},        // boundary out of the vocabulary
      {2, 3, -1, 0, 0},
      {2, 3, 5, 0, 97},       // tokens 97, 98, 99: [M] committed
      {2, 3, 5, 0, -2},       // a negative token
  };
  for (const auto& b : bad) {
    make_record(o, b[0], b[1], b[2], b[3], b[4]);
    CHECK(code_of([&] { read_accept(o, B, V, MASK, &ro); }, "invalid") == SSB_EHIP);
  }
}

struct Seq : PageList, SeqState {
  std::unique_ptr<int32_t[]> table;
};

static void check_tables(const std::vector<Seq*>& seqs, const PageStack& pool) {
  std::set<int> seen(pool.free_pages.begin(), pool.free_pages.end());
  CHECK((int)seen.size() == pool.n_free());
  size_t held = 0;
  for (const Seq* s : seqs) {
    held += s->pages.size();
    CHECK((int)s->pages.size() <= s->max_pages);
    for (size_t i = 0; i < s->pages.size(); ++i) {
      CHECK(s->pages[i] >= 0 && s->pages[i] < pool.n_pages);
      CHECK(s->table[i] == s->pages[i]);
      CHECK(seen.insert(s->pages[i]).second);   // no page held twice or both held and free
    }
  }
  CHECK((int)(held + pool.n_free()) == pool.n_pages);
}

// Rounds, rewinds and resets on four sequences over one pool, in the order the engine makes them:
// ensure the window (p + B + 2 positions), read the records, commit, trim past the next window.
static void check_random_rounds() {
  std::mt19937 rng(12345);
  const int B = 32, V = 60000, MASK = 59999, n_pages = 160;
  PageStack pool;
  pool.init(n_pages);
  std::vector<std::unique_ptr<Seq>> own;
  std::vector<Seq*> seqs;
  for (int i = 0; i < 4; ++i) {
    own.emplace_back(new Seq());
    Seq* s = own.back().get();
    s->init(600 + 100 * i);
    s->table.reset(new int32_t[s->max_pages]);
    seqs.push_back(s);
  }
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int rounds = 0, nokv = 0, rejected = 0;
  for (int it = 0; it < 200000; ++it) {
    const int op = uni(0, 99);
    if (op < 5) {   // reset one sequence
      Seq* s = seqs[uni(0, 3)];
      s->trim(pool, 0);
      s->seq_len = 0;
      s->x0 = -1;
    } else if (op < 12) {   // prefill one sequence that has none
      Seq* s = seqs[uni(0, 3)];
      if (s->x0 >= 0) continue;
      const int P = uni(1, 200);
      if (code_of([&] { s->ensure(pool, P, s->table.get()); }) != SSB_OK) { ++nokv; continue; }
      s->seq_len = P;
      s->x0 = uni(0, V - 2);
    } else if (op < 20) {   // rewind
      Seq* s = seqs[uni(0, 3)];
      const int n = uni(-2, s->seq_len + 2);
      const int32_t x0 = uni(-1, V);
      if (code_of([&] { check_rewind(*s, n, x0, V, MASK); }) == SSB_OK) {
        s->seq_len = n;
        s->x0 = x0;
        s->trim(pool, n + B + 2);
      }
    } else {   // a batched round over the prefilled sequences
      std::vector<Seq*> batch;
      for (Seq* s : seqs)
        if (s->x0 >= 0 && uni(0, 1)) batch.push_back(s);
      if (batch.empty()) continue;
      const int R = (int)batch.size();
      bool ok = true;
      for (Seq* s : batch)
        if (code_of([&] { s->ensure(pool, s->seq_len + B + 2, s->table.get()); }) != SSB_OK) ok = false;
      if (!ok) { ++nokv; continue; }   // the engine fails the call; pages taken so far stay held
      std::vector<int32_t> recs((size_t)R * kOutStride, 0);
      std::vector<int> p(R);
      const int bad = uni(0, 9) == 0 ? uni(0, R - 1) : -1;
      for (int r = 0; r < R; ++r) {
        p[r] = batch[r]->seq_len;
        const int A = uni(0, B);
        const int n = std::min(A + 2, uni(1, B + 2));
        make_record(&recs[(size_t)r * kOutStride], r == bad ? B + 1 : A, n, uni(0, V - 2), 0, uni(0, 100));
      }
      std::vector<SeqState> before;
      std::vector<size_t> pages_before;
      for (Seq* s : batch) {
        before.push_back(*s);
        pages_before.push_back(s->pages.size());
      }
      std::vector<RoundOut> out(R);
      const int rc = code_of([&] { commit_batch(batch.data(), R, pool, p.data(), recs.data(), B, V, MASK, out.data()); });
      if (bad >= 0) {
        CHECK(rc == SSB_EHIP);
        ++rejected;
        for (int r = 0; r < R; ++r) {
          CHECK(batch[r]->seq_len == before[r].seq_len && batch[r]->x0 == before[r].x0);
          CHECK(batch[r]->pages.size() == pages_before[r]);
        }
      } else {
        CHECK(rc == SSB_OK);
        ++rounds;
        for (int r = 0; r < R; ++r) {
          CHECK(batch[r]->seq_len == p[r] + out[r].A + 2);
          CHECK((int)batch[r]->pages.size() == std::min(pages_for(batch[r]->seq_len + B + 2), (int)pages_before[r]));
        }
      }
      // rounds that reach a sequence's max_tokens end it, as a caller's decode would
      for (Seq* s : batch)
        if (s->seq_len + B + 2 > s->max_tokens) {
          s->trim(pool, 0);
          s->seq_len = 0;
          s->x0 = -1;
        }
    }
    if (it % 97 == 0) check_tables(seqs, pool);
  }
  check_tables(seqs, pool);
  CHECK(rounds > 10000 && rejected > 1000 && nokv > 0);
  std::printf("random rounds: %d committed, %d rejected records, %d pool/capacity refusals\n", rounds, rejected, nokv);
}

int main() {
#ifdef SSB_HOST_CHECK_CONTROL
  PageStack pool;
  pool.init(8);
  PageList pl;
  pl.init(64);   // 4 pages
  std::unique_ptr<int32_t[]> table(new int32_t[pl.max_pages - 1]);
  pl.ensure(pool, 64, table.get());   // writes table[3]: one past the end
  std::printf("control: no overflow reported\n");
  return 0;
#else
  check_errors();
  check_configs();
  check_pages_basic();
  check_rewinds();
  check_records();
  check_random_rounds();
  std::printf("host checks passed: %d checks\n", g_checks);
  return 0;
#endif
}
