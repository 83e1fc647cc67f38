// Host-side exercise of the library under AddressSanitizer and
// UndefinedBehaviorSanitizer: the decode and shared-pass planners, workspace
// sizing, argument checks that return before any launch, pool sizing near the
// integer limits, status strings, and the block manager / continuous-batching
// scheduler on seeded random workloads. Built from host-only objects (no
// device code is compiled or run); the test prints "ok" and exits 0, and any
// sanitizer report aborts the process with a non-zero status.
#include <pkv.h>
#include <pkv_sched.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <set>
#include <vector>

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, long long a = 0, long long b = 0) {
  if (!ok) {
    fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, a, b);
    ++g_fail;
  }
}

// splitmix64: a small counter-based generator for the random workloads
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int in(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }
};

void planners() {
  const int seqs[] = {1, 7, 64, 192, 1024, 1025, 65535, 65536, 70000};
  const int ctxs[] = {1, 15, 16, 17, 512, 2048, 8191, 8192, 100000, 1 << 20};
  const int hds[] = {16, 32, 64, 128, 256, 96};
  const int bss[] = {1, 16, 64, 256};
  const int kvs[] = {1, 3, 8};
  const int reps[] = {1, 3, 8, 9};
  for (int dt = 0; dt < 3; ++dt)
    for (int hd : hds)
      for (int bs : bss)
        for (int kv : kvs)
          for (int rep : reps)
            for (int s : seqs)
              for (int c : ctxs) {
                pkv_pool_desc pool = {1 << 16, bs, kv, hd, dt};
                const int hq = kv * rep;
                const int32_t part = pkv_decode_partition(s, c, &pool);
                const size_t ws = pkv_decode_workspace_bytes(s, hq, c, part, &pool);
                const size_t ws0 = pkv_decode_workspace_bytes(s, hq, c, 0, &pool);
                expect(ws < ((size_t)1 << 50), "decode workspace bound", (long long)ws);
                (void)ws0;
                for (int groups : {0, 1, 4}) {
                  const int mg = groups ? (s + groups - 1) / groups : 0;
                  const size_t wss = pkv_decode_shared_workspace_bytes(
                      s, hq, c, groups, mg, c / 2, c, 0, &pool);
                  expect(wss < ((size_t)1 << 50), "shared workspace bound", (long long)wss);
                }
              }
  // degenerate sizes must be refused or give 0, never crash
  pkv_pool_desc bad = {0, 0, 0, 0, 7};
  (void)pkv_decode_partition(-1, -5, &bad);
  (void)pkv_decode_workspace_bytes(-1, -1, -1, -1, &bad);
  (void)pkv_decode_partition(1, 1, nullptr);
  (void)pkv_decode_workspace_bytes(1, 1, 1, 0, nullptr);
  (void)pkv_decode_shared_workspace_bytes(1, 1, 1, 1, 1, 1, 1, 0, nullptr);
}

// Every call below is invalid in one argument and must return an error
// before anything is launched.
void argument_checks() {
  alignas(16) static char dev[4096];   // stands in for device memory; never touched
  void* p = dev;
  int32_t* ip = reinterpret_cast<int32_t*>(dev);
  pkv_pool_desc pool = {64, 16, 8, 128, PKV_BF16};
  pkv_pool_desc badbs = {64, 12, 8, 128, PKV_BF16};
  pkv_pool_desc badhd = {64, 16, 8, 96, PKV_BF16};
  pkv_pool_desc baddt = {64, 16, 8, 128, 5};
  size_t ws = 1 << 20;

  expect(pkv_decode(nullptr, 4, 64, p, p, &pool, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_NULL, "decode null q");
  expect(pkv_decode(p, 4, 64, p, p, nullptr, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_NULL, "decode null pool");
  expect(pkv_decode(p, 4, 64, p, p, &baddt, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_DTYPE, "decode dtype");
  expect(pkv_decode(p, -1, 64, p, p, &pool, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_SHAPE, "decode negative seqs");
  expect(pkv_decode(p, 4, 60, p, p, &pool, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_SHAPE, "decode heads not a multiple");
  expect(pkv_decode(p, 4, 64, p, p, &pool, ip, 4, ip, 65, 0.1f, 0, p, p, ws, nullptr) ==
             PKV_ERR_SHAPE, "decode context past the table");
  expect(pkv_decode(p, 4, 64, p, p, &badbs, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) !=
             PKV_OK, "decode block size");
  expect(pkv_decode(p, 4, 64, p, p, &badhd, ip, 4, ip, 64, 0.1f, 0, p, p, ws, nullptr) !=
             PKV_OK, "decode head_dim");
  expect(pkv_decode(p, 4, 64, p, p, &pool, ip, 4, ip, 64, 0.1f, 0, dev + 1, p, ws, nullptr) ==
             PKV_ERR_ALIGN, "decode misaligned out");
  expect(pkv_decode(p, 4, 64, p, p, &pool, ip, 64, ip, 1024, 0.1f, 0, p, p, 16, nullptr) ==
             PKV_ERR_WORKSPACE, "decode small workspace");
  expect(pkv_decode_step(p, nullptr, p, 4, 64, p, p, &pool, ip, 4, ip, 64, 0.1f, 0, p, p, ws,
                         nullptr) == PKV_ERR_NULL, "step null k_new");
  expect(pkv_decode_step_noalloc(p, p, p, 4, 64, p, p, &pool, ip, 4, ip, 65, 0.1f, 0, p,
                                 nullptr) == PKV_ERR_SHAPE, "noalloc context past the table");
  expect(pkv_write(nullptr, p, ip, 4, p, p, &pool, nullptr) == PKV_ERR_NULL, "write null");
  expect(pkv_write(p, p, ip, -4, p, p, &pool, nullptr) == PKV_ERR_SHAPE, "write negative");
  expect(pkv_slot_mapping(ip, 0, 1, ip, ip, 4, 16, 64, ip, nullptr) == PKV_ERR_SHAPE,
         "slot mapping no table");
  expect(pkv_prefill(p, ip, 4, 64, 16, 64, p, p, &pool, ip, 4, ip, 128, 0.1f, p, nullptr) ==
             PKV_ERR_SHAPE, "prefill context past the table");
  expect(pkv_decode_shared(p, 4, 64, p, p, &pool, ip, 4, ip, 64, nullptr, ip, 2, 2, 32, 32,
                           0.1f, 0, p, p, ws, nullptr) == PKV_ERR_NULL, "shared null groups");
  // a long error message is cut, never overrun
  const char* e = pkv_last_error();
  expect(e != nullptr && strlen(e) < 4096, "last error");
}

void statuses() {
  // 0..15 is the value range of the enum (its enumerators are 0..8); values
  // outside it cannot be formed in C++ without undefined behaviour
  for (int s = 0; s < 16; ++s) {
    const char* t = pkv_status_string((pkv_status)s);
    expect(t != nullptr && strlen(t) > 0, "status string", s);
  }
  expect(pkv_abi_version() == PKV_ABI_VERSION, "abi version");
}

void pool_sizing() {
  const int64_t big = INT64_MAX;
  const int32_t dims[] = {0, 1, 16, 128, INT32_MAX};
  for (int32_t a : dims)
    for (int32_t b : dims)
      for (int32_t c : dims) (void)pkv_block_bytes(a, b, c, 128, 2);
  (void)pkv_block_bytes(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);
  (void)pkv_block_bytes(-1, 16, 8, 128, 2);
  const int64_t frees[] = {0, 1, 1 << 30, (int64_t)24 << 30, big / 2, big};
  const double utils[] = {0.0, 0.5, 0.9, 1.0, 1.5, -1.0};
  const int64_t bbs[] = {0, 1, 32768, 524288, big};
  for (int64_t f : frees)
    for (double u : utils)
      for (int64_t bb : bbs)
        for (int32_t mml : {0, 1, 2048, INT32_MAX}) {
          int64_t nb = -7, req = -7;
          (void)pkv_plan_pool(f, big, u, f / 3, bb, 16, mml, &nb, &req);
          (void)pkv_plan_pool(f, f, u, 0, bb, 1, mml, &nb, &req);
        }
  int64_t nb, req;
  expect(pkv_plan_pool(1 << 30, 1 << 30, 0.9, 0, 524288, 16, 2048, nullptr, &req) != PKV_OK,
         "plan pool null");
  expect(pkv_plan_pool((int64_t)24 << 30, (int64_t)24 << 30, 0.9, 0, 524288, 16, 2048, &nb,
                       &req) == PKV_OK, "plan pool 24 GiB");
}

// Random workloads through the scheduler: small pools force preemption; the
// step lists must stay consistent with the pool (no block held twice).
void scheduler(uint64_t seed) {
  Rng r{seed};
  int64_t preemptions = 0, done = 0;
  for (int trial = 0; trial < 40; ++trial) {
    const int bs = 1 << r.in(0, 5);
    const int nblocks = r.in(1, 96);
    const int max_batch = r.in(1, 16);
    const int maxb = r.in(1, 64);
    const int continuous = r.in(0, 1);
    pkv_sched* s = pkv_sched_create(nblocks, bs, max_batch, continuous, maxb);
    expect(s != nullptr, "create");
    if (!s) continue;
    const int nreq = r.in(0, 40);
    int accepted = -1;   // an id the scheduler took
    for (int i = 0; i < nreq; ++i) {
      const int prompt = r.in(1, 3 * bs + 5);
      const int max_new = r.in(1, 4 * bs + 3);
      const int stop = r.in(1, max_new);
      if (pkv_sched_submit(s, i, prompt, max_new, stop) == PKV_OK && accepted < 0) accepted = i;
    }
    // a duplicate id and bad sizes are refused
    if (accepted >= 0) expect(pkv_sched_submit(s, accepted, 1, 1, 1) != PKV_OK, "duplicate rid");
    expect(pkv_sched_submit(s, 100000, 0, 1, 1) != PKV_OK, "empty prompt");
    std::vector<int32_t> prid(max_batch), plen(max_batch), ptab((size_t)max_batch * maxb);
    std::vector<int32_t> drid(max_batch), dpos(max_batch), dtab((size_t)max_batch * maxb);
    pkv_sched_step_out none;
    memset(&none, 0, sizeof(none));
    expect(pkv_sched_step(s, &none) == PKV_ERR_NULL, "step without arrays");
    for (int step = 0; step < 20000 && pkv_sched_pending(s) > 0; ++step) {
      pkv_sched_step_out out;
      memset(&out, 0, sizeof(out));
      out.prefill_rid = prid.data();
      out.prefill_len = plen.data();
      out.prefill_tables = ptab.data();
      out.decode_rid = drid.data();
      out.decode_pos = dpos.data();
      out.decode_tables = dtab.data();
      const pkv_status st = pkv_sched_step(s, &out);
      if (st != PKV_OK) break;   // a request larger than the whole pool
      std::set<int32_t> held;
      auto check_rows = [&](int n, const int32_t* len, const int32_t* tables, bool decode) {
        for (int i = 0; i < n; ++i) {
          const int tokens = decode ? len[i] + 1 : len[i];
          const int need = (tokens + bs - 1) / bs;
          expect(need <= maxb, "table width", need, maxb);
          for (int b = 0; b < need && b < maxb; ++b) {
            const int32_t id = tables[(size_t)i * maxb + b];
            expect(id >= 0 && id < nblocks, "block id range", id, nblocks);
            expect(held.insert(id).second, "block held twice", id);
          }
        }
      };
      check_rows(out.num_decode, out.decode_pos, out.decode_tables, true);
      // every admitted request is running, so it also has a decode row
      for (int i = 0; i < out.num_prefill; ++i)
        expect(std::find(out.decode_rid, out.decode_rid + out.num_decode, out.prefill_rid[i]) !=
                   out.decode_rid + out.num_decode, "prefill row decoded", out.prefill_rid[i]);
    }
    pkv_sched_stats st;
    expect(pkv_sched_get_stats(s, &st) == PKV_OK, "stats");
    preemptions += st.preemptions;
    done += st.requests_done;
    std::vector<int32_t> run(st.steps + 1);
    std::vector<int64_t> a(st.steps + 1), b(st.steps + 1), c(st.steps + 1);
    expect(pkv_sched_history(s, run.data(), a.data(), b.data(), c.data(), st.steps + 1) ==
               st.steps, "history length");
    pkv_sched_destroy(s);
  }
  // the workloads reached the interesting paths
  expect(preemptions > 0, "some preemption", preemptions);
  expect(done > 0, "some requests retired", done);
  expect(pkv_sched_create(0, 16, 1, 1, 1) == nullptr, "create zero blocks");
  pkv_sched_destroy(nullptr);
}

}  // namespace

int main() {
  planners();
  argument_checks();
  statuses();
  pool_sizing();
  scheduler(12345);
  scheduler(987654321);
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("ok\n");
  return 0;
}
