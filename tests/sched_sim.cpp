// Discrete-event simulation of the layer stream's ordering protocol.
//
// The SlotScheduler of the library (the same header the runtime compiles)
// is driven by an executor that models the two device streams: every stream
// runs its operations in order, a wait blocks until the event version that
// was last recorded when the wait was enqueued has completed (the semantics
// of hipStreamWaitEvent / hipEventSynchronize), and copies and layer
// computations take random durations.  After a run of whole training steps
// the simulation checks, for every layer computation (and every LM-head
// chunk read through a slot), that its slot held the right record, copied
// completely before the read began, and that no copy into the slot
// overlapped the read; and it reports the number of record copies.
//
// usage: sched_sim <scenario> <n_layers> <n_slots> <steps> <seed>
//   scenario: sft (F B), sfth (F H B: LM head streamed through two slots),
//             dpo (F F B: separate reference pass), dpoh (F H F H B)
// prints "loads <n>" and exits 0, or prints the first violation and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <random>
#include <string>
#include <vector>

#include "../layer_streamed_nf4_double_amd/csrc/sched.h"

using lsn::MAX_SLOTS;

namespace {

enum { WAIT = 0, RECORD = 1, WRITE = 2, READ = 3 };
constexpr int COPY = 0, COMPUTE = 1;
constexpr int NEV = 2 * MAX_SLOTS;  // copy_done[s] = s, slot_free[s] = MAX_SLOTS + s

struct Op {
  int kind, ev;
  uint64_t ver;
  double dur;
  int slot, tag;
};
struct Interval {
  double a, b;
  int slot, tag;
};

struct Sim {
  std::mt19937_64 rng;
  std::deque<Op> q[2];
  double t[2] = {0, 0};
  uint64_t recorded[NEV] = {};          // versions enqueued per event
  std::vector<double> done_at[NEV];     // completion time of each version
  std::vector<Interval> writes, reads;

  explicit Sim(uint64_t seed) : rng(seed) {}
  double uniform(double lo, double hi) {
    return std::uniform_real_distribution<double>(lo, hi)(rng);
  }
  void wait(int stream, int ev) { q[stream].push_back({WAIT, ev, recorded[ev], 0, -1, 0}); }
  void record(int stream, int ev) { q[stream].push_back({RECORD, ev, ++recorded[ev], 0, -1, 0}); }
  void work(int stream, int kind, int slot, int tag, double dur) {
    q[stream].push_back({kind, -1, 0, dur, slot, tag});
  }
  // one operation of a stream; false if it is blocked or idle
  bool step(int s) {
    if (q[s].empty()) return false;
    const Op o = q[s].front();
    if (o.kind == WAIT) {
      if (o.ver > 0) {  // a wait on an event never recorded is a no-op
        if (done_at[o.ev].size() < o.ver) return false;
        t[s] = std::max(t[s], done_at[o.ev][o.ver - 1]);
      }
    } else if (o.kind == RECORD) {
      done_at[o.ev].push_back(t[s]);
    } else {
      const double a = t[s];
      t[s] += o.dur;
      (o.kind == WRITE ? writes : reads).push_back({a, t[s], o.slot, o.tag});
    }
    q[s].pop_front();
    return true;
  }
  void run() {
    for (;;) {
      bool any = false;
      while (step(COPY)) any = true;
      while (step(COMPUTE)) any = true;
      if (!any) return;
    }
  }
  // host blocks until the last recorded version of ev has completed
  bool host_wait(int ev) {
    const uint64_t v = recorded[ev];
    run();
    return done_at[ev].size() >= v;
  }
};

struct SimExec {
  Sim* sim;
  int copy_wait_free(int s) {
    sim->wait(COPY, MAX_SLOTS + s);
    return 0;
  }
  int host_wait_copy(int s) { return sim->host_wait(s) ? 0 : 90; }
  int copy_record(int layer, int s, int next) {
    (void)next;
    sim->work(COPY, WRITE, s, layer, sim->uniform(0.5, 3.0));
    sim->record(COPY, s);
    return 0;
  }
  int compute_wait_copy(int s) {
    sim->wait(COMPUTE, s);
    return 0;
  }
  int compute_free(int s) {
    sim->record(COMPUTE, MAX_SLOTS + s);
    return 0;
  }
};

int fail(const char* fmt, int a, int b, int c) {
  printf("FAIL: ");
  printf(fmt, a, b, c);
  printf("\n");
  return 1;
}

// A pass over the layers in `order`: each position is computed between
// layer_begin and layer_end (reads = 2 for the fused reference + policy pair).
int pass(lsn::SlotScheduler<SimExec>& sch, SimExec& x, const std::vector<int>& order) {
  int st = sch.begin(x, order);
  if (st) return fail("begin_pass status %d (%d %d)", st, 0, 0);
  for (size_t i = 0; i < order.size(); ++i) {
    int s = -1;
    st = sch.layer_begin(x, &s);
    if (st) return fail("layer_begin status %d at position %d (%d)", st, (int)i, 0);
    x.sim->work(COMPUTE, READ, s, order[i], x.sim->uniform(0.1, 4.0));
    st = sch.layer_end(x);
    if (st) return fail("layer_end status %d at position %d (%d)", st, (int)i, 0);
  }
  return 0;
}

// The LM head with its table streamed through two slots in `chunks` chunks
// (tags -1, -2, ...), each chunk copied while the previous one is read.
int head(lsn::SlotScheduler<SimExec>& sch, SimExec& x, int chunks) {
  int hs[2];
  if (sch.foreign_slots(2, hs)) return fail("no head slots (%d %d %d)", 0, 0, 0);
  auto copy = [&](int i) {
    const int s = hs[i & 1];
    int st = sch.foreign_prepare(x, s);
    if (st) return st;
    x.sim->work(COPY, WRITE, s, -1 - i, x.sim->uniform(0.2, 1.5));
    x.sim->record(COPY, s);
    sch.foreign_copied(s);
    return 0;
  };
  for (int i = 0; i < std::min(chunks, 2); ++i)
    if (copy(i)) return fail("head copy %d (%d %d)", i, 0, 0);
  for (int i = 0; i < chunks; ++i) {
    const int s = hs[i & 1];
    if (sch.foreign_acquire(x, s)) return fail("head acquire %d (%d %d)", i, 0, 0);
    x.sim->work(COMPUTE, READ, s, -1 - i, x.sim->uniform(0.1, 2.0));
    if (sch.foreign_release(x, s)) return fail("head release %d (%d %d)", i, 0, 0);
    if (i + 2 < chunks && copy(i + 2)) return fail("head copy %d (%d %d)", i + 2, 0, 0);
  }
  return 0;
}

// Every read saw its record: the last write into its slot that ended before
// the read began carries the read's tag, and no write into the slot overlaps
// the read.
int check(const Sim& sim) {
  for (const Interval& r : sim.reads) {
    int last = -1;
    for (size_t w = 0; w < sim.writes.size(); ++w) {
      const Interval& c = sim.writes[w];
      if (c.slot != r.slot) continue;
      if (c.a < r.b && c.b > r.a)
        return fail("a copy of tag %d into slot %d overlaps the read of tag %d", c.tag, r.slot,
                    r.tag);
      if (c.b <= r.a && (last < 0 || c.b >= sim.writes[last].b)) last = (int)w;
    }
    if (last < 0) return fail("read of tag %d in slot %d before any copy (%d)", r.tag, r.slot, 0);
    if (sim.writes[last].tag != r.tag)
      return fail("read of tag %d found tag %d in slot %d", r.tag, sim.writes[last].tag, r.slot);
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s sft|sfth|dpo|dpoh n_layers n_slots steps seed\n", argv[0]);
    return 2;
  }
  const std::string scen = argv[1];
  const int L = atoi(argv[2]), n = atoi(argv[3]), steps = atoi(argv[4]);
  Sim sim(strtoull(argv[5], nullptr, 10));
  SimExec x{&sim};
  lsn::SlotScheduler<SimExec> sch;
  sch.init(n);
  std::vector<int> fwd(L), bwd(L);
  for (int i = 0; i < L; ++i) {
    fwd[i] = i;
    bwd[i] = L - 1 - i;
  }
  const bool with_head = scen == "sfth" || scen == "dpoh";
  const bool dpo = scen == "dpo" || scen == "dpoh";
  for (int k = 0; k < steps; ++k) {
    if (dpo) {  // reference forward (and its head pass)
      if (pass(sch, x, fwd)) return 1;
      if (with_head && head(sch, x, 3)) return 1;
    }
    if (pass(sch, x, fwd)) return 1;
    if (with_head && head(sch, x, 3)) return 1;
    if (pass(sch, x, bwd)) return 1;
  }
  sim.run();
  if (!sim.q[0].empty() || !sim.q[1].empty()) return fail("streams blocked (%d %d %d)", 0, 0, 0);
  if (check(sim)) return 1;
  printf("loads %llu\n", (unsigned long long)sch.loads);
  return 0;
}
