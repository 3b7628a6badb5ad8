// Host replay of the attention forward kernels' index arithmetic (test
// infrastructure).  For each workload it builds the library's own plan,
// then runs the kernels' index functions (attn_index.h) for every work
// item, tile, query slot and DMA lane, and checks:
//  * the persistent walk hands every work item to exactly one workgroup;
//  * every tile lies inside the item's key rows, full tiles are whole and
//    every item of the persistent walk ends with a boundary tile;
//  * every key a valid query row may see, within the item's key split,
//    lies in some tile of the item, the full tiles hold only keys that every
//    valid row sees, and the key splits of a query tile partition the keys;
//  * every global element offset the kernels form (Q and O rows, K and V rows
//    of each DMA lane, log-sum-exp entries, split partials) stays inside its
//    tensor, in 64-bit arithmetic, including workloads past 2^31 elements;
//  * the DMA rings of the persistent and split-key walks: replaying each
//    workgroup's sequence of issues, waits and reads, every tile a step
//    reads has landed and still owns its stage.
// Prints "ok" and returns 0 when every check held.  With the argument
// "no-stand-in" it replays the ring without the stand-in loads the walk
// issues once its stream is exhausted, and must then report failures.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>
#include <vector>

#include "attn_index.h"
#include "internal.h"

using namespace bda;

static long long failures = 0;
#define CHECK(cond, ...)                                                        \
  do {                                                                          \
    if (!(cond)) {                                                              \
      if (failures < 20) {                                                      \
        fprintf(stderr, "%s:%d: %s: ", __FILE__, __LINE__, #cond);              \
        fprintf(stderr, __VA_ARGS__);                                           \
        fprintf(stderr, "\n");                                                  \
      }                                                                         \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

// Keys row qrow may see (geometry.h), as two spans.
static void spans(const AttnIndex& a, int L, int qrow, Span& A, Span& C) {
  row_spans(a.mode, L, a.n, a.blk, qrow, A, C);
}

template <int D>
static void dma_lanes(const AttnIndex& a, int pair, int t0, int t1, size_t kv_rows, const char* what) {
  // the kernel's DMA: wavefront w loads runs w*DJ + q; lane i fills bytes
  // 1024 run + 16 i of the stage, i.e. key r, chunk c = fwd_at(...); a short
  // tile repeats its last key
  constexpr int CPR = D / 8, TCH = kBN * CPR, NT = 512, DJ = TCH >= NT ? TCH / NT : 1;
  for (int w = 0; w < 8; ++w)
    for (int q = 0; q < DJ; ++q) {
      const int run = w * DJ + q;
      if (run * 64 >= TCH) continue;
      for (int lane = 0; lane < 64; ++lane) {
        int r, c;
        fwd_at<D>(1024 * run + 16 * lane, r, c);
        CHECK(r >= 0 && r < kBN && c >= 0 && c < CPR, "%s: lane %d of run %d names key %d chunk %d", what, lane,
              run, r, c);
        CHECK(fwd_off<D>(r, c) == 1024 * run + 16 * lane, "%s: layout not inverted", what);
        const int key = t0 + imin(r, t1 - 1 - t0);
        const size_t elem = attn_kv_elem<D>(a, pair, key) + 8 * (size_t)c;
        CHECK(key >= t0 && key < t1 && elem + 8 <= kv_rows * D, "%s: DMA of key %d (tile [%d,%d)) past K/V", what,
              key, t0, t1);
      }
    }
}

static bool g_stand_in = true;

// The persistent walk's DMA ring as attn.hip runs it.  Stream tile t of a
// workgroup (its items' tiles in order) goes to stage t % 4, issued three
// steps ahead; the prologue issues three and waits for all.  An item starts
// by waiting for every load (its Q operands).  Every step first issues the
// next stream tile into the stage the previous step freed; once the stream
// is exhausted a fast step issues the stand-in there instead and a
// boundary step nothing.  Fast step i of an item reads stream tiles i and
// i + 1 (the next tile's K); a boundary step reads tile i, after waiting
// for every load when it had nothing to issue.  Every step ends by waiting
// for all loads but the newest, then the barrier.  After an item's last step
// its epilogue uses the stage of that step's tile as scratch.
static void ring_replay(const AttnIndex& a, const int32_t* kv_len, long long grid, const char* what) {
  for (long long wg = 0; wg < grid; ++wg) {
    std::vector<Geom> items;
    long long T = 0;
    for (int r = 0;; ++r) {
      const int idx = attn_item_of(a, (int)grid, (int)wg, r);
      if (idx < 0) break;
      Geom gm;
      attn_geom(a, kWalkPersistent, kv_len, idx, gm);
      items.push_back(gm);
      T += gm.nt;
    }
    std::vector<long long> issue_of((size_t)T, -1);
    long long owner[4] = {-1, -1, -1, -1};   // issue that last wrote each stage
    long long issued = 0, landed = 0, next_tile = 0;
    // issue at stream position pos; returns whether it was a stream tile
    auto issue = [&](long long pos, bool stand_in) -> bool {
      if (next_tile < T) {
        CHECK(next_tile == pos, "%s: wg %lld issues tile %lld at position %lld", what, wg, next_tile, pos);
        issue_of[(size_t)next_tile++] = issued;
        owner[pos & 3] = issued++;
        return true;
      }
      if (stand_in && g_stand_in) owner[pos & 3] = issued++;
      return false;
    };
    auto read = [&](long long t) {
      const bool ok = t < T && issue_of[(size_t)t] >= 0 && issue_of[(size_t)t] < landed &&
                      owner[t & 3] == issue_of[(size_t)t];
      CHECK(ok, "%s: wg %lld reads stream tile %lld of %lld before it landed or after its stage was reused", what,
            wg, t, T);
    };
    auto settle = [&]() { landed = std::max(landed, issued - 1); };
    for (int k = 0; k < 3; ++k) issue(k, false);
    landed = issued;
    long long sp = 0;
    for (const Geom& gm : items) {
      landed = issued;
      for (int i = 0; i < gm.nf; ++i) {
        issue(sp + i + 3, true);
        read(sp + i);
        read(sp + i + 1);
        settle();
      }
      for (int i = gm.nf; i < gm.nt; ++i) {
        if (!issue(sp + i + 3, false)) landed = issued;
        read(sp + i);
        settle();
      }
      sp += gm.nt;
      // the item's epilogue stages O in the ring stage of its last tile
      // (waves 0..3) until a barrier that precedes the next step's issue:
      // no issue since that tile may have gone into that stage
      const long long last = sp - 1;
      CHECK(last < 0 ? owner[3] == -1 : owner[last & 3] == issue_of[(size_t)last],
            "%s: wg %lld: the stage of stream tile %lld was reissued before the item's epilogue", what, wg, last);
    }
  }
}

// The split-key walk's DMA ring as attn.hip runs it, for one item: tile t
// goes to stage t % 5.  The prologue of a long walk (more than 8 tiles)
// issues up to four and waits for all; that of a short walk issues tile 0,
// waits for it (the statement that loads Q), then issues tiles 1 .. 3.
// Step i first issues the next tile (into the stage of tile i - 1, which the
// step before finished), reads tile i, then waits until tile i + 1 has
// landed (up to three tiles issued after it stay in flight) and the
// barrier.
static void split_ring_replay(const Geom& gm, const char* what, int idx) {
  const int nt = gm.nt;
  long long owner[5] = {-1, -1, -1, -1, -1};
  long long issued = 0, landed = 0;
  auto issue = [&]() {
    if (issued >= nt) return;
    owner[issued % 5] = issued;
    ++issued;
  };
  auto read = [&](long long t) {
    const bool ok = t < nt && t < landed && owner[t % 5] == t;
    CHECK(ok, "%s: split item %d reads tile %lld of %d before it landed or after its stage was reused", what, idx,
          t, nt);
  };
  if (nt <= 8) {
    issue();
    landed = issued;
    for (int k = 1; k < 4; ++k) issue();
  } else {
    for (int k = 0; k < 4; ++k) issue();
    landed = issued;
  }
  for (int i = 0; i < nt; ++i) {
    issue();
    read(i);
    const long long newer = std::min(3LL, std::max(0LL, issued - 1 - (i + 1)));
    landed = std::max(landed, issued - newer);
  }
}

template <int D>
static void replay(const char* what, int B, int Hq, int Hkv, int L, int block, int mode, const int32_t* kv_len,
                   int cus = 256) {
  AttnPlan p;
  const char* why = "";
  if (attn_make_plan(B, Hq, Hkv, L, D, block, mode, &p, &why)) {
    CHECK(false, "%s: no plan (%s)", what, why);
    return;
  }
  AttnIndex a;
  attn_fill_index(p, &a);
  const int walk = p.stages == 4 ? kWalkPersistent : (p.stages == 5 ? kWalkSplit : kWalkRegs);
  const int nw = p.nw;
  const size_t q_rows = (size_t)B * Hq * p.Sq, kv_rows = (size_t)B * Hkv * p.Sk;
  // the persistent walk's item order covers every item once
  if (walk == kWalkPersistent) {
    int ppx = 0;
    const long long grid = attn_persistent_grid(p, cus, &ppx);
    a.pairs_per_xcd = ppx;
    std::vector<int> seen((size_t)a.n_items, 0);
    for (long long wg = 0; wg < grid; ++wg)
      for (int r = 0;; ++r) {
        const int idx = attn_item_of(a, (int)grid, (int)wg, r);
        if (idx < 0) break;
        CHECK(idx < a.n_items, "%s: item %d of %d", what, idx, a.n_items);
        if (idx < a.n_items) ++seen[(size_t)idx];
      }
    for (int i = 0; i < a.n_items; ++i) CHECK(seen[(size_t)i] == 1, "%s: item %d taken %d times", what, i, seen[(size_t)i]);
    ring_replay(a, kv_len, grid, what);
  }
  for (int idx = 0; idx < a.n_items; ++idx) {
    Geom gm;
    attn_geom(a, walk, kv_len, idx, gm);
    const int b = gm.pair / Hkv, g = gm.pair % Hkv;
    CHECK(gm.pair >= 0 && gm.pair < B * Hkv && gm.qt >= 0 && gm.qt < a.n_qtiles && gm.split >= 0 &&
              gm.split < a.n_splits, "%s: item %d: pair %d qt %d split %d", what, idx, gm.pair, gm.qt, gm.split);
    const int Lrow = mode == kHybrid ? L : gm.L;
    CHECK(mode == kHybrid || (gm.L >= a.n && gm.L <= L), "%s: item %d: key count %d", what, idx, gm.L);
    // tiles: each of the ranges F, R1, R2 is covered by consecutive tiles
    // without gaps; the staged keys are then the union of the three ranges
    Span ranges[3] = {gm.F, gm.R1, gm.R2};
    int j = 0;
    for (int rg = 0; rg < 3; ++rg) {
      int next = ranges[rg].lo;
      const int count = rg == 0 ? gm.nf : (rg == 1 ? gm.n1 : gm.nt - gm.nf - gm.n1);
      for (int t = 0; t < count; ++t, ++j) {
        int t0, t1;
        attn_tile(gm, j, t0, t1);
        CHECK(t0 >= 0 && t0 < t1 && t1 <= p.Sk && t1 - t0 <= kBN, "%s: item %d tile %d = [%d,%d)", what, idx, j,
              t0, t1);
        CHECK(rg > 0 || t1 - t0 == kBN, "%s: item %d: short full tile %d", what, idx, j);
        CHECK(t0 == next, "%s: item %d: tile %d starts at %d, not %d", what, idx, j, t0, next);
        next = t1;
        if (idx % 7 == 0 || j == 0 || j == gm.nt - 1) dma_lanes<D>(a, gm.pair, t0, t1, kv_rows, what);
      }
      CHECK(count == 0 || next == ranges[rg].hi, "%s: item %d: range %d [%d,%d) tiled to %d", what, idx, rg,
            ranges[rg].lo, ranges[rg].hi, next);
    }
    // keys of [k0, k1) outside the staged ranges
    auto uncovered = [&](int k0, int k1) -> int {
      for (int k = k0; k < k1;) {
        bool moved = false;
        for (int rg = 0; rg < 3; ++rg)
          if (ranges[rg].hi > ranges[rg].lo && k >= ranges[rg].lo && k < ranges[rg].hi) {
            k = ranges[rg].hi;
            moved = true;
          }
        if (!moved) return k;
      }
      return -1;
    };
    CHECK(walk != kWalkPersistent || gm.nt == 0 || gm.nt > gm.nf, "%s: item %d ends with a full tile", what, idx);
    if (walk == kWalkSplit) split_ring_replay(gm, what, idx);
    // query slots: bounds, key coverage, full tiles visible to every valid row
    const int halves = mode == kHybrid ? 2 : 1;
    const int slots = mode == kHybrid ? (nw / 2) * 32 : (walk == kWalkSplit ? nw / 2 : nw) * 32;
    const int lo = mode == kHybrid ? 0 : gm.split * a.split_keys;
    const int hi = mode == kHybrid ? p.Sk : imin(Lrow, lo + a.split_keys);
    for (int h = 0; h < halves; ++h)
      for (int s = 0; s < slots; ++s) {
        int qrow, head;
        const bool valid = attn_slot(a, h, s, gm.qt, g, qrow, head);
        if (!valid) continue;
        CHECK(qrow >= 0 && qrow < p.Sq && head >= 0 && head < Hq && head / (Hq / Hkv) == g,
              "%s: item %d slot %d: row %d head %d", what, idx, s, qrow, head);
        const size_t qe = attn_q_elem<D>(a, b, head, qrow);
        CHECK(attn_q_row(a, b, head, qrow) < q_rows && qe + D <= q_rows * D, "%s: Q/O element %zu of %zu", what,
              qe, q_rows * D);
        if (p.n_splits > 1) {
          const size_t pe = attn_part_elem<D>(a, gm.split, b, head, qrow);
          CHECK(pe + D <= (size_t)p.n_splits * B * Hq * p.n * D, "%s: partial element %zu", what, pe);
        }
        Span A, C;
        spans(a, Lrow, qrow, A, C);
        const int ua = uncovered(imax(A.lo, lo), imin(A.hi, hi)), uc = uncovered(imax(C.lo, lo), imin(C.hi, hi));
        CHECK(ua < 0 && uc < 0, "%s: item %d row %d: key %d not staged", what, idx, qrow, ua >= 0 ? ua : uc);
        // the full tiles [F.lo, F.hi) lie inside A or inside C (which may touch)
        const bool fa = gm.F.hi <= gm.F.lo || (gm.F.lo >= A.lo && gm.F.hi <= A.hi) ||
                        (gm.F.lo >= C.lo && gm.F.hi <= C.hi) ||
                        (A.hi == C.lo && gm.F.lo >= A.lo && gm.F.hi <= C.hi) ||
                        (C.hi == A.lo && gm.F.lo >= C.lo && gm.F.hi <= A.hi);
        CHECK(fa, "%s: item %d row %d: full tiles [%d,%d) not all visible", what, idx, qrow, gm.F.lo, gm.F.hi);
      }
  }
  // the key splits of every (pair, query tile) partition [0, Sk)
  if (mode != kHybrid) {
    CHECK((long long)a.n_splits * a.split_keys >= L && (long long)(a.n_splits - 1) * a.split_keys < L,
          "%s: %d splits of %d keys for L = %d", what, a.n_splits, a.split_keys, L);
  }
}

int main(int argc, char** argv) {
  if (argc > 1 && std::string(argv[1]) == "no-stand-in") g_stand_in = false;
  // the benchmark's workloads
  replay<128>("training form B4 L2048 b32", 4, 32, 8, 2048, 32, kHybrid, nullptr);
  replay<128>("prefill B2 n=L=4096", 2, 32, 8, 4096, 4096, kCausal, nullptr);
  replay<128>("decode B32 KV4124 n28", 32, 32, 8, 4124, 28, kDecode, nullptr);
  replay<128>("verify B16 KV8220 n28", 16, 32, 8, 8220, 28, kCausal, nullptr);
  replay<128>("training form, 160 compute units", 4, 32, 8, 2048, 32, kHybrid, nullptr, 160);
  // canvas step and speculative step: per-row lengths below, at and past the capacity
  {
    const int32_t kl[2] = {4096 + 28, 4352 + 9};
    replay<128>("canvas decode B2 cap4352 n28", 2, 32, 8, 4352, 28, kDecode, kl);
    int32_t kl16[16];
    for (int b = 0; b < 16; ++b) kl16[b] = 8192 - 37 * b + 28 - (b == 3 ? 9000 : 0);
    replay<128>("speculative decode B16 cap8444 n28", 16, 32, 8, 8444, 28, kDecode, kl16);
    replay<128>("speculative causal B16 cap8444 n28", 16, 32, 8, 8444, 28, kCausal, kl16);
  }
  // multi-item and ragged cases at every head dim, small cases, every mode
  replay<128>("hybrid B4 L1024 b32", 4, 32, 8, 1024, 32, kHybrid, nullptr);
  replay<64>("hybrid d64 B4 L2048 b32", 4, 32, 8, 2048, 32, kHybrid, nullptr);
  replay<32>("hybrid d32 B4 L1536 b28", 4, 32, 8, 1536, 28, kHybrid, nullptr);
  replay<128>("hybrid B3 L1000 b7", 3, 32, 8, 1000, 7, kHybrid, nullptr);
  replay<64>("causal d64 B4 n=L=2100", 4, 32, 8, 2100, 2100, kCausal, nullptr);
  for (int L = 1; L <= 300; L += 23)
    for (int blk = 1; blk <= L; blk += 1 + L / 4) {
      replay<128>("hybrid small", 1, 8, 2, L, blk, kHybrid, nullptr);
      replay<64>("hybrid small d64", 2, 6, 2, L, blk, kHybrid, nullptr);
      replay<32>("decode small d32", 2, 4, 1, L, blk, kDecode, nullptr);
      replay<128>("causal small", 1, 32, 8, L, blk, kCausal, nullptr);
    }
  // past 2^31 elements: decode over an 80 x 32768-key cache (K and V 2.7 G
  // elements each), and a 32-bit-overflowing query tensor
  replay<128>("decode B80 KV32768 n28", 80, 32, 8, 32768, 28, kDecode, nullptr);
  replay<128>("causal B80 KV32768 n1024", 80, 32, 8, 32768, 1024, kCausal, nullptr);
  if (failures) {
    fprintf(stderr, "%lld failed checks\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
