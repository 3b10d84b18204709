// Slot scheduler of the layer stream: which layer record goes into which
// device slot, and when each stream waits for which event.  Host logic only
// (no HIP here): the runtime drives it with an executor that issues HIP
// stream operations, and a CPU test drives the same code with a simulated
// two-stream executor that checks the ordering it produces.
//
// The mechanism ("Soup: Fine-Tune an 8B Model on a 4 GB GPU", section "The
// Core Idea: Layer Streaming"): the frozen base is copied to the GPU one
// decoder layer at a time, on a stream of its own, as the forward or the
// backward pass reaches the layer.  Here a pass is an ordered list of layers;
// n device slots (2: a double buffer) hold records.  The scheduler keeps the
// next n positions of the pass resident or in flight:
//   - a position whose layer already sits in a slot reuses it (no copy);
//   - otherwise it takes a slot that holds no record of the window, the one
//     freed earliest, and the copy stream waits for that slot's slot_free
//     event (recorded by the compute stream after the slot's last reader)
//     before copying into it, then records copy_done;
//   - the compute stream waits for copy_done of its slot before a layer and
//     records slot_free after it.
// Before queueing a copy into a slot the host waits for the previous copy
// into that slot, so at most one copy per slot is queued at any time.
//
// Executor interface (each call returns 0, or a nonzero status that the
// scheduler returns unchanged):
//   int copy_wait_free(int s);   copy stream waits for the last slot_free[s]
//   int host_wait_copy(int s);   host blocks until the last copy_done[s]
//   int copy_record(int layer, int s, int next);
//                                copy stream copies layer's record into slot
//                                s and records copy_done[s] (next: the layer
//                                the pass needs after it and that is not in a
//                                slot, a read-ahead hint; -1 none)
//   int compute_wait_copy(int s);  compute stream waits for copy_done[s]
//   int compute_free(int s);       compute stream records slot_free[s]
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace lsn {

constexpr int MAX_SLOTS = 4;

// Status returned when no slot can take a position (cannot happen while the
// window is no wider than the slot count; kept as a guard).
constexpr int SCHED_NO_SLOT = -1;

template <class Exec>
class SlotScheduler {
 public:
  int nslots = 2;
  int slot_layer[MAX_SLOTS];  // record held or on its way (-1: none or foreign data)
  bool freed[MAX_SLOTS];      // slot_free[s] has been recorded at least once
  bool copied[MAX_SLOTS];     // copy_done[s] has been recorded at least once
  uint64_t free_seq[MAX_SLOTS];  // when the slot was last released (0: never used)
  uint64_t seq = 0;
  std::vector<int> order;    // layers of the current pass, in pass order
  std::vector<int> slot_of;  // slot of each position once assigned (-1: not yet)
  size_t pos = 0;            // next position to compute
  uint64_t loads = 0;        // record copies issued

  void init(int n) {
    nslots = n < 1 ? 1 : n > MAX_SLOTS ? MAX_SLOTS : n;
    for (int s = 0; s < MAX_SLOTS; ++s) {
      slot_layer[s] = -1;
      freed[s] = copied[s] = false;
      free_seq[s] = 0;
    }
    order.clear();
    slot_of.clear();
    pos = 0;
  }

  bool in_pass() const { return pos < order.size(); }

  // Starts a pass over `ord` and queues the copies of its first positions.
  int begin(Exec& x, const std::vector<int>& ord) {
    order = ord;
    slot_of.assign(ord.size(), -1);
    pos = 0;
    return fill(x);
  }

  // A slot holding `layer` now holds stale data (the record was rewritten).
  void forget(int layer) {
    for (int s = 0; s < nslots; ++s)
      if (slot_layer[s] == layer) slot_layer[s] = -1;
  }

  // Compute side of position pos: its record is resident or in flight (fill),
  // the compute stream waits for its copy; *slot receives the slot.
  int layer_begin(Exec& x, int* slot) {
    int st = fill(x);
    if (st) return st;
    const int s = slot_of[pos];
    st = x.compute_wait_copy(s);
    if (st) return st;
    *slot = s;
    return 0;
  }

  // After the last kernel of position pos: the slot is released and the
  // window moves on (queueing the copy of the position that enters it).
  int layer_end(Exec& x) {
    const int s = slot_of[pos];
    int st = x.compute_free(s);
    if (st) return st;
    freed[s] = true;
    free_seq[s] = ++seq;
    pos += 1;
    return fill(x);
  }

  // Slots for data that is not a layer record (the LM-head chunks streamed
  // through the slots): the `count` slots released earliest, whose records
  // the next pass needs last.  Outside a pass only.
  int foreign_slots(int count, int* out) const {
    bool taken[MAX_SLOTS] = {};
    for (int i = 0; i < count; ++i) {
      int best = -1;
      for (int s = 0; s < nslots; ++s)
        if (!taken[s] && (best < 0 || free_seq[s] < free_seq[best])) best = s;
      if (best < 0) return SCHED_NO_SLOT;
      taken[best] = true;
      out[i] = best;
    }
    return 0;
  }

  // Before the caller copies foreign data into slot s on the copy stream:
  // the copy stream waits for the slot's last reader, the host for the
  // slot's previous copy.  The caller then enqueues the copy and calls
  // foreign_copied(s) after recording copy_done[s].
  int foreign_prepare(Exec& x, int s) {
    if (freed[s]) {
      int st = x.copy_wait_free(s);
      if (st) return st;
    }
    if (copied[s]) {
      int st = x.host_wait_copy(s);
      if (st) return st;
    }
    slot_layer[s] = -1;
    return 0;
  }
  void foreign_copied(int s) { copied[s] = true; }
  // Before the compute stream reads foreign data from slot s.
  int foreign_acquire(Exec& x, int s) { return x.compute_wait_copy(s); }
  // After the compute stream has read foreign data from slot s.
  int foreign_release(Exec& x, int s) {
    int st = x.compute_free(s);
    if (st) return st;
    freed[s] = true;
    free_seq[s] = ++seq;
    return 0;
  }

 private:
  bool holds_window_record(int s, size_t end, size_t except) const {
    for (size_t j = pos; j < end; ++j) {
      if (j == except) continue;
      if (slot_of[j] == s) return true;
      if (slot_of[j] < 0 && slot_layer[s] == order[j]) return true;
    }
    return false;
  }

  // Positions pos .. pos + nslots - 1: each reuses the slot holding its
  // layer, or gets a copy into a slot that holds no record of the window.
  int fill(Exec& x) {
    const size_t end = order.size() < pos + nslots ? order.size() : pos + nslots;
    for (size_t i = pos; i < end; ++i) {
      if (slot_of[i] >= 0) continue;
      const int layer = order[i];
      int s = -1;
      for (int q = 0; q < nslots; ++q)
        if (slot_layer[q] == layer) s = q;
      if (s < 0) {
        for (int q = 0; q < nslots; ++q)
          if (!holds_window_record(q, end, i) && (s < 0 || free_seq[q] < free_seq[s])) s = q;
        if (s < 0) return SCHED_NO_SLOT;
        // read-ahead hint: the pass's next layer, unless it sits in a slot
        int next = -1;
        if (i + 1 < order.size()) {
          next = order[i + 1];
          for (int q = 0; q < nslots; ++q)
            if (slot_layer[q] == next) next = -1;
        }
        if (freed[s]) {
          int st = x.copy_wait_free(s);
          if (st) return st;
        }
        if (copied[s]) {
          int st = x.host_wait_copy(s);
          if (st) return st;
        }
        slot_layer[s] = -1;
        int st = x.copy_record(layer, s, next);
        if (st) return st;
        copied[s] = true;
        slot_layer[s] = layer;
        loads += 1;
      }
      slot_of[i] = s;
    }
    return 0;
  }
};

}  // namespace lsn
