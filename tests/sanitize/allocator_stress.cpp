// Stress driver for the host block allocator, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_allocator_sanitized.py (CPU only).
//
// Runs seeded random sequences of allocator calls through the C ABI, keeps an
// independent shadow of every reference count, of the host swap pool and of
// every table, and checks after each call that the library agrees; error
// paths (OOM, double free, bad ids, unknown sequences, lookups past the
// allocated blocks, operations on swapped-out sequences) must leave the state
// unchanged.  At the end every sequence is freed and every count must be 0
// with the free list a permutation of 0..N-1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

#define REQUIRE(cond)                                                              \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      std::fprintf(stderr, "FAILED %s at line %d (last error: %s)\n", #cond, __LINE__, \
                   pkv_last_error());                                              \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

namespace {

struct Shadow {
  std::vector<int> refs;
  struct Seq {
    int32_t id;
    std::vector<int32_t> blocks;  // host ids while swapped out
    int tokens;
    int min_window;
    bool swapped;
  };
  std::vector<Seq> seqs;
  std::vector<int32_t> host_free;  // the next host block to leave is at the back
};

void check_counts(pkv_allocator* a, const Shadow& sh, int nb) {
  int free_blocks = 0;
  for (int b = 0; b < nb; ++b) {
    int rc = -1;
    REQUIRE(pkv_ref_count(a, b, &rc) == PKV_OK);
    REQUIRE(rc == sh.refs[b]);
    free_blocks += rc == 0;
  }
  int nf = -1;
  REQUIRE(pkv_num_free(a, &nf) == PKV_OK);
  REQUIRE(nf == free_blocks);
}

void run(unsigned seed, int nb, int bs, int ops) {
  std::mt19937 rng(seed);
  pkv_allocator* a = nullptr;
  REQUIRE(pkv_allocator_create(nb, bs, &a) == PKV_OK);
  Shadow sh;
  sh.refs.assign(nb, 0);
  const int nhb = nb / 2;
  REQUIRE(pkv_allocator_set_host_pool(a, nhb) == PKV_OK);
  for (int h = 0; h < nhb; ++h) sh.host_free.push_back(h);
  std::vector<int32_t> slots(4 * bs + 8), ids(nb + 1);
  int32_t cow[2];
  for (int op = 0; op < ops; ++op) {
    const int kind = static_cast<int>(rng() % 9);
    if (kind == 0 || sh.seqs.empty()) {  // new sequence
      int32_t s = -1;
      REQUIRE(pkv_seq_create(a, &s) == PKV_OK);
      sh.seqs.push_back({s, {}, 0, 0, false});
    } else if (kind == 1 || kind == 2) {  // append tokens (may need CoW or fail with OOM)
      auto& q = sh.seqs[rng() % sh.seqs.size()];
      const int n = static_cast<int>(rng() % (3 * bs + 1));
      int ncow = -1;
      const int rc = pkv_seq_append_tokens(a, q.id, n, slots.data(), cow, 1, &ncow);
      if (q.swapped) {
        REQUIRE(rc == PKV_ERR_INVALID_ARG);
      } else if (rc == PKV_OK) {
        for (int t = 0; t < n; ++t) {
          const int pos = q.tokens + t;
          if (pos % bs == 0) {
            REQUIRE(slots[t] % bs == 0);
            const int32_t b = slots[t] / bs;
            REQUIRE(sh.refs[b] == 0);
            sh.refs[b] = 1;
            q.blocks.push_back(b);
          } else if (t == 0 && ncow == 1) {
            REQUIRE(cow[0] == q.blocks.back());
            REQUIRE(sh.refs[cow[1]] == 0 && sh.refs[cow[0]] > 1);
            --sh.refs[cow[0]];
            sh.refs[cow[1]] = 1;
            q.blocks.back() = cow[1];
          }
          REQUIRE(slots[t] == q.blocks.back() * bs + pos % bs);
        }
        q.tokens += n;
      } else {
        REQUIRE(rc == PKV_ERR_OOM);
      }
    } else if (kind == 3) {  // fork
      auto parent = sh.seqs[rng() % sh.seqs.size()];
      int32_t c = -1;
      if (parent.swapped) {
        REQUIRE(pkv_seq_fork(a, parent.id, &c) == PKV_ERR_INVALID_ARG);
      } else {
        REQUIRE(pkv_seq_fork(a, parent.id, &c) == PKV_OK);
        for (int32_t b : parent.blocks)
          if (b >= 0) ++sh.refs[b];
        sh.seqs.push_back({c, parent.blocks, parent.tokens, parent.min_window, false});
      }
    } else if (kind == 4) {  // free a sequence
      const size_t i = rng() % sh.seqs.size();
      REQUIRE(pkv_seq_free(a, sh.seqs[i].id) == PKV_OK);
      for (int32_t b : sh.seqs[i].blocks) {
        if (b < 0) continue;
        if (sh.seqs[i].swapped)
          sh.host_free.push_back(b);
        else
          --sh.refs[b];
      }
      sh.seqs.erase(sh.seqs.begin() + static_cast<long>(i));
    } else if (kind == 8) {  // swap out or in, whichever applies
      auto& q = sh.seqs[rng() % sh.seqs.size()];
      int held = 0;
      for (int32_t b : q.blocks) held += b >= 0;
      std::vector<int32_t> pairs(2 * (q.blocks.size() + 1));
      int np = -1;
      const int cap = static_cast<int>(q.blocks.size());
      if (!q.swapped) {
        const int rc = pkv_seq_swap_out(a, q.id, pairs.data(), cap, &np);
        REQUIRE(np == held);
        if (held > static_cast<int>(sh.host_free.size())) {
          REQUIRE(rc == PKV_ERR_OOM);
        } else {
          REQUIRE(rc == PKV_OK);
          int k = 0;
          for (int32_t& b : q.blocks) {
            if (b < 0) continue;
            REQUIRE(pairs[2 * k] == b && pairs[2 * k + 1] == sh.host_free.back());
            sh.host_free.pop_back();
            --sh.refs[b];
            b = pairs[2 * k + 1];
            ++k;
          }
          q.swapped = true;
        }
      } else {
        int nfree = 0;
        REQUIRE(pkv_num_free(a, &nfree) == PKV_OK);
        const int rc = pkv_seq_swap_in(a, q.id, pairs.data(), cap, &np);
        REQUIRE(np == held);
        if (held > nfree) {
          REQUIRE(rc == PKV_ERR_OOM);
        } else {
          REQUIRE(rc == PKV_OK);
          int k = 0;
          for (int32_t& h : q.blocks) {
            if (h < 0) continue;
            const int32_t d = pairs[2 * k + 1];
            REQUIRE(pairs[2 * k] == h && sh.refs[d] == 0);
            sh.refs[d] = 1;
            sh.host_free.push_back(h);
            h = d;
            ++k;
          }
          q.swapped = false;
        }
      }
      int hf = -1, sw = -1;
      REQUIRE(pkv_host_num_free(a, &hf) == PKV_OK && hf == static_cast<int>(sh.host_free.size()));
      REQUIRE(pkv_seq_is_swapped(a, q.id, &sw) == PKV_OK && sw == (q.swapped ? 1 : 0));
    } else if (kind == 5) {  // errors that must change nothing
      int32_t out = 0;
      REQUIRE(pkv_seq_physical_block(a, sh.seqs[0].id,
                                     static_cast<int>(sh.seqs[0].blocks.size()) * bs, &out) ==
              (sh.seqs[0].swapped ? PKV_ERR_INVALID_ARG : PKV_ERR_INDEX));
      REQUIRE(pkv_seq_free(a, -5) == PKV_ERR_INVALID_ARG);
      int32_t bad = nb;
      REQUIRE(pkv_free(a, &bad, 1) == PKV_ERR_INVALID_ARG);
      int nfree = 0;
      REQUIRE(pkv_num_free(a, &nfree) == PKV_OK);
      REQUIRE(pkv_allocate(a, nfree + 1, ids.data()) == PKV_ERR_OOM);
      for (int b = 0; b < nb; ++b) {
        if (sh.refs[b] == 0) {
          int32_t id = b;
          REQUIRE(pkv_free(a, &id, 1) == PKV_ERR_DOUBLE_FREE);
          REQUIRE(pkv_incref(a, &id, 1) == PKV_ERR_INVALID_ARG);
          break;
        }
      }
    } else if (kind == 7) {  // sliding-window trim
      auto& q = sh.seqs[rng() % sh.seqs.size()];
      const int w = 1 + static_cast<int>(rng() % (3 * bs));
      std::vector<int32_t> rel(q.blocks.size() + 1);
      int nrel = -1;
      if (q.swapped) {
        REQUIRE(pkv_seq_trim_window(a, q.id, w, rel.data(), static_cast<int>(rel.size()), &nrel) ==
                PKV_ERR_INVALID_ARG);
        check_counts(a, sh, nb);
        continue;
      }
      REQUIRE(pkv_seq_trim_window(a, q.id, w, rel.data(), static_cast<int>(rel.size()), &nrel) ==
              PKV_OK);
      const int first_kept = std::max(0, q.tokens - w) / bs;
      int k = 0;
      for (int j = 0; j < first_kept; ++j) {
        if (q.blocks[j] < 0) continue;
        REQUIRE(rel[k] == q.blocks[j]);
        --sh.refs[q.blocks[j]];
        q.blocks[j] = -1;
        ++k;
      }
      REQUIRE(nrel == k);
      q.min_window = q.min_window ? std::min(q.min_window, w) : w;
    } else {  // raw block ops: allocate, share, copy-on-write, release
      int32_t b = -1;
      if (pkv_allocate(a, 1, &b) == PKV_OK) {
        REQUIRE(sh.refs[b] == 0);
        sh.refs[b] = 1;
        REQUIRE(pkv_incref(a, &b, 1) == PKV_OK);
        ++sh.refs[b];
        int32_t nb2 = -1;
        int copied = -1;
        const int rc = pkv_copy_on_write(a, b, &nb2, &copied);
        if (rc == PKV_OK) {
          REQUIRE(copied == 1 && nb2 != b && sh.refs[nb2] == 0);
          --sh.refs[b];
          sh.refs[nb2] = 1;
          REQUIRE(pkv_copy_on_write(a, nb2, &nb2, &copied) == PKV_OK && copied == 0);
          REQUIRE(pkv_free(a, &nb2, 1) == PKV_OK);
          --sh.refs[nb2];
        } else {
          REQUIRE(rc == PKV_ERR_OOM);
          REQUIRE(pkv_free(a, &b, 1) == PKV_OK);
          --sh.refs[b];
        }
        REQUIRE(pkv_free(a, &b, 1) == PKV_OK);
        --sh.refs[b];
      }
    }
    check_counts(a, sh, nb);
  }
  // Export tables for the resident sequences and check them against the shadow.
  std::vector<const Shadow::Seq*> res;
  for (auto& q : sh.seqs)
    if (!q.swapped) res.push_back(&q);
  if (!res.empty()) {
    int mb = 1;
    std::vector<int32_t> sid;
    for (auto* q : res) {
      sid.push_back(q->id);
      if (static_cast<int>(q->blocks.size()) > mb) mb = static_cast<int>(q->blocks.size());
    }
    std::vector<int32_t> tables(sid.size() * mb), lens(sid.size());
    REQUIRE(pkv_export_block_tables(a, sid.data(), static_cast<int>(sid.size()), mb, -1,
                                    tables.data(), lens.data()) == PKV_OK);
    for (size_t i = 0; i < sid.size(); ++i) {
      REQUIRE(lens[i] == res[i]->tokens);
      for (int j = 0; j < mb; ++j)
        REQUIRE(tables[i * mb + j] ==
                (j < static_cast<int>(res[i]->blocks.size()) ? res[i]->blocks[j] : -1));
    }
    // each table is valid for decode with the smallest window it was trimmed to
    for (size_t i = 0; i < sid.size(); ++i) {
      int bad_s = 0, bad_b = 0;
      REQUIRE(pkv_validate_tables(tables.data() + i * mb, lens.data() + i, 1, mb, bs, nb,
                                  res[i]->min_window, &bad_s, &bad_b) == PKV_OK);
    }
  }
  for (auto& q : sh.seqs) {
    REQUIRE(pkv_seq_free(a, q.id) == PKV_OK);
    for (int32_t b : q.blocks) {
      if (b < 0) continue;
      if (q.swapped)
        sh.host_free.push_back(b);
      else
        --sh.refs[b];
    }
  }
  check_counts(a, sh, nb);
  int hf = -1;
  REQUIRE(pkv_host_num_free(a, &hf) == PKV_OK && hf == nhb);
  std::vector<int32_t> fl(nb);
  int n = 0;
  REQUIRE(pkv_free_list(a, fl.data(), nb, &n) == PKV_OK && n == nb);
  std::vector<char> seen(nb, 0);
  for (int i = 0; i < nb; ++i) {
    REQUIRE(fl[i] >= 0 && fl[i] < nb && !seen[fl[i]]);
    seen[fl[i]] = 1;
  }
  REQUIRE(pkv_allocator_destroy(a) == PKV_OK);
}

}  // namespace

int main(int argc, char** argv) {
  const int seeds = argc > 1 ? std::atoi(argv[1]) : 20;
  for (int s = 0; s < seeds; ++s) run(1000u + s, 8 + s * 3, s % 2 ? 16 : 4, 3000);
  std::printf("allocator stress ok: %d seeds\n", seeds);
  return 0;
}
