// Task-graph builder, static validator and protocol simulator (host only).
#include "graph.h"

#include <algorithm>
#include <cstdio>
#include <map>
#include <random>
#include <sstream>
#include <tuple>

namespace mk {

namespace {

std::string fmt(const char* f, long a = 0, long b = 0, long c = 0, long d = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

}  // namespace

int auto_split(int max_seq) {
  (void)max_seq;
  return 64;  // one 16-position block per wave of a 4-wave attention workgroup (head_dim 128)
}

std::string build_graph(const GraphConfig& c, Graph& g) {
  if (c.B != 1) return "batch > 1 is not supported by this graph builder";
  if (c.L < 1 || c.H < 8 || c.nq < 1 || c.nkv < 1 || c.F < 8 || c.V < 1 || c.max_seq < 1 || c.ncu < 1)
    return "graph: non-positive dimension";
  if (c.hd != 64 && c.hd != 128) return "graph: head_dim must be 64 or 128";
  if (c.nq % c.nkv) return "graph: n_q_heads must be a multiple of n_kv_heads";
  if (c.nq / c.nkv > kMaxGqa) return "graph: more than 8 query heads per KV head";
  if (c.H % 8 || c.F % 8 || (c.nq * c.hd) % 8) return "graph: hidden, ffn and n_q_heads*head_dim must be multiples of 8";
  if (c.split < 1 || c.split > kMaxSplit) return "graph: attention split must be in [1, 4096]";
  g = Graph();
  g.cfg = c;
  g.nsplit = (c.max_seq + c.split - 1) / c.split;
  const int half = c.hd / 2;

  int n_events = 0;
  auto new_event = [&]() { return n_events++; };
  std::vector<int> ev_x(c.L + 1, -1), ev_qkv(c.L), ev_mrg(c.L), ev_xmid(c.L), ev_h(c.L);
  std::vector<std::vector<int>> ev_att(c.L, std::vector<int>(c.B * c.nkv));
  for (int l = 0; l < c.L; ++l) {
    ev_qkv[l] = new_event();
    for (auto& e : ev_att[l]) e = new_event();
    ev_mrg[l] = new_event();
    ev_xmid[l] = new_event();
    ev_h[l] = new_event();
    ev_x[l + 1] = new_event();
  }
  const int ev_lm = new_event();
  if (n_events >= kNone16) return "graph: too many events";

  auto add = [&](uint8_t type, int layer, int in_ev, int out_ev, uint16_t key, int b, int a0, int a1, int a2, int a3) {
    Task t{};
    t.type = type;
    t.page = kNone8;
    t.layer = (uint16_t)layer;
    t.in_event = in_ev < 0 ? kNone16 : (uint16_t)in_ev;
    t.out_event = out_ev < 0 ? kNone16 : (uint16_t)out_ev;
    t.stage = key;
    t.batch = (uint16_t)b;
    t.id = (uint32_t)g.tasks.size();
    t.a0 = a0; t.a1 = a1; t.a2 = a2; t.a3 = a3;
    g.tasks.push_back(t);
    g.stage_of.push_back((int)g.stage_begin.size() - 1);
  };
  auto begin_stage = [&](uint8_t type) {
    g.stage_begin.push_back((int)g.tasks.size());
    g.stage_type.push_back(type);
  };

  for (int l = 0; l < c.L; ++l) {
    const int in_x = l == 0 ? -1 : ev_x[l];
    begin_stage(TT_QKV);
    for (int b = 0; b < c.B; ++b) {
      for (int m = 0; m < 2; ++m) {  // q, k: one task per RoPE pair (i, i + hd/2)
        const int heads = m == 0 ? c.nq : c.nkv;
        for (int hh = 0; hh < heads; ++hh)
          for (int i = 0; i < half; ++i)
            add(TT_QKV, l, in_x, ev_qkv[l], stage_key(SK_ATTN_NORM, l), b, m, hh * c.hd + i, 2, half);
      }
      const int vrows = c.nkv * c.hd;
      for (int r = 0; r < vrows; r += kRowsQkv)
        add(TT_QKV, l, in_x, ev_qkv[l], stage_key(SK_ATTN_NORM, l), b, 2, r, std::min(kRowsQkv, vrows - r), 0);
    }
    begin_stage(TT_ATTN);
    for (int b = 0; b < c.B; ++b)
      for (int grp = 0; grp < c.nkv; ++grp)
        for (int s = 0; s < g.nsplit; ++s)
          add(TT_ATTN, l, ev_qkv[l], ev_att[l][b * c.nkv + grp], 0, b, grp, s, 0, 0);
    begin_stage(TT_MERGE);
    for (int b = 0; b < c.B; ++b)
      for (int grp = 0; grp < c.nkv; ++grp)
        add(TT_MERGE, l, ev_att[l][b * c.nkv + grp], ev_mrg[l], 0, b, grp, 0, 0, 0);
    begin_stage(TT_O);
    for (int b = 0; b < c.B; ++b)
      for (int r = 0; r < c.H; r += kRowsO)
        add(TT_O, l, ev_mrg[l], ev_xmid[l], stage_key(SK_O_IN, l), b, 0, r, std::min(kRowsO, c.H - r), 0);
    begin_stage(TT_GU);
    for (int b = 0; b < c.B; ++b)
      for (int r = 0; r < c.F; r += kRowsGuPerMatrix)
        add(TT_GU, l, ev_xmid[l], ev_h[l], stage_key(SK_FFN_NORM, l), b, 0, r, std::min(kRowsGuPerMatrix, c.F - r), 0);
    begin_stage(TT_DOWN);
    for (int b = 0; b < c.B; ++b)
      for (int r = 0; r < c.H; r += kRowsDown)
        add(TT_DOWN, l, ev_h[l], ev_x[l + 1], stage_key(SK_H, l), b, 0, r, std::min(kRowsDown, c.H - r), 0);
  }
  begin_stage(TT_LM);
  for (int b = 0; b < c.B; ++b)
    for (int r = 0; r < c.V; r += kRowsLm)
      add(TT_LM, c.L, ev_x[c.L], ev_lm, stage_key(SK_FINAL_NORM, c.L), b, 0, r, std::min(kRowsLm, c.V - r), 0);
  begin_stage(TT_ARGMAX);
  add(TT_ARGMAX, c.L, ev_lm, -1, 0, 0, 0, 0, 0, 0);
  g.stage_begin.push_back((int)g.tasks.size());

  // Placement: each stage's tasks go round-robin over the CUs, starting where
  // the previous stage stopped, so per-CU work stays within one task per stage.
  const int nt = (int)g.tasks.size();
  g.cu_of.assign(nt, 0);
  int rr = 0;
  for (size_t s = 0; s + 1 < g.stage_begin.size(); ++s) {
    const int b0 = g.stage_begin[s], b1 = g.stage_begin[s + 1];
    for (int i = b0; i < b1; ++i) g.cu_of[i] = (rr + (i - b0)) % c.ncu;
    rr = (rr + (b1 - b0)) % c.ncu;
  }
  g.queues.assign(c.ncu, {});
  for (int i = 0; i < nt; ++i) g.queues[g.cu_of[i]].push_back(i);  // ids are topological

  // Aggregated signals: consecutive tasks of a queue with the same output event
  // form a run that signals the event once; an event fires after all runs.
  g.event_count.assign(n_events, 0);
  for (int cu = 0; cu < c.ncu; ++cu) {
    auto& q = g.queues[cu];
    int run_no = 0;
    for (size_t i = 0; i < q.size();) {
      Task& t0 = g.tasks[q[i]];
      size_t j = i;
      while (j < q.size() && g.tasks[q[j]].out_event == t0.out_event) ++j;
      for (size_t k = i; k < j; ++k) {
        g.tasks[q[k]].local_slot = (uint16_t)(run_no % kLocalSlots);
        g.tasks[q[k]].local_count = (uint16_t)(j - i);
      }
      if (t0.out_event != kNone16) g.event_count[t0.out_event] += 1;
      ++run_no;
      i = j;
    }
    // LDS pages: alternate between the two pages at every change of staged input.
    uint16_t last = 0;
    uint8_t page = 1;
    for (int id : q) {
      Task& t = g.tasks[id];
      if (!t.stage) continue;
      if (t.stage != last) { page ^= 1; last = t.stage; }
      t.page = page;
    }
  }
  for (auto& t : g.tasks)
    if (t.in_event != kNone16) t.in_count = g.event_count[t.in_event];

  g.flat.clear();
  g.queue_off.assign(c.ncu + 1, 0);
  for (int cu = 0; cu < c.ncu; ++cu) {
    g.queue_off[cu] = (int32_t)g.flat.size();
    for (int id : g.queues[cu]) g.flat.push_back(g.tasks[id]);
  }
  g.queue_off[c.ncu] = (int32_t)g.flat.size();
  return "";
}

// ---------------------------------------------------------------------------
// Static validation
namespace {

enum Buf { B_Q, B_K, B_V, B_PART, B_AOUT, B_XMID, B_H, B_X, B_LM, B_OUT };
struct Region {
  int buf, l, b, grp;  // key
  int lo, hi;          // [lo, hi) within the key's buffer
};
using Key = std::tuple<int, int, int, int>;
inline Key key_of(const Region& r) { return Key(r.buf, r.l, r.b, r.grp); }

void task_regions(const Graph& g, const Task& t, std::vector<Region>& rd, std::vector<Region>& wr) {
  const auto& c = g.cfg;
  const int G = c.nq / c.nkv, l = t.layer, b = t.batch;
  rd.clear();
  wr.clear();
  switch (t.type) {
    case TT_QKV: {
      if (l > 0) rd.push_back({B_X, l, b, 0, 0, c.H});
      const int buf = t.a0 == 0 ? B_Q : t.a0 == 1 ? B_K : B_V;
      if (t.a3) {
        wr.push_back({buf, l, b, 0, t.a1, t.a1 + t.a2 / 2});
        wr.push_back({buf, l, b, 0, t.a1 + t.a3, t.a1 + t.a3 + t.a2 / 2});
      } else {
        wr.push_back({buf, l, b, 0, t.a1, t.a1 + t.a2});
      }
      break;
    }
    case TT_ATTN:
      rd.push_back({B_Q, l, b, 0, t.a0 * G * c.hd, (t.a0 + 1) * G * c.hd});
      rd.push_back({B_K, l, b, 0, t.a0 * c.hd, (t.a0 + 1) * c.hd});
      rd.push_back({B_V, l, b, 0, t.a0 * c.hd, (t.a0 + 1) * c.hd});
      wr.push_back({B_PART, l, b, t.a0, t.a1, t.a1 + 1});
      break;
    case TT_MERGE:
      rd.push_back({B_PART, l, b, t.a0, 0, g.nsplit});
      wr.push_back({B_AOUT, l, b, 0, t.a0 * G * c.hd, (t.a0 + 1) * G * c.hd});
      break;
    case TT_O:
      rd.push_back({B_AOUT, l, b, 0, 0, c.nq * c.hd});
      if (l > 0) rd.push_back({B_X, l, b, 0, t.a1, t.a1 + t.a2});
      wr.push_back({B_XMID, l, b, 0, t.a1, t.a1 + t.a2});
      break;
    case TT_GU:
      rd.push_back({B_XMID, l, b, 0, 0, c.H});
      wr.push_back({B_H, l, b, 0, t.a1, t.a1 + t.a2});
      break;
    case TT_DOWN:
      rd.push_back({B_H, l, b, 0, 0, c.F});
      rd.push_back({B_XMID, l, b, 0, t.a1, t.a1 + t.a2});
      wr.push_back({B_X, l + 1, b, 0, t.a1, t.a1 + t.a2});
      break;
    case TT_LM:
      rd.push_back({B_X, c.L, b, 0, 0, c.H});
      wr.push_back({B_LM, 0, b, 0, 0, 1});  // accumulated (max), many writers
      break;
    case TT_ARGMAX:
      for (int bb = 0; bb < c.B; ++bb) rd.push_back({B_LM, 0, bb, 0, 0, 1});
      wr.push_back({B_OUT, 0, 0, 0, 0, c.B});
      break;
  }
}

struct Write {
  int lo, hi, task;
};

}  // namespace

std::string validate_graph(const Graph& g) {
  const auto& c = g.cfg;
  const int nt = (int)g.tasks.size();
  const int ne = (int)g.event_count.size();
  // 1. every task exactly once; 2. queue order topological
  std::vector<int> seen(nt, 0);
  for (int cu = 0; cu < c.ncu; ++cu) {
    int last_stage = -1;
    for (int id : g.queues[cu]) {
      if (id < 0 || id >= nt) return "queue holds an invalid task id";
      if (seen[id]++) return fmt("task %ld queued twice", id);
      if (g.stage_of[id] < last_stage) return fmt("CU %ld queue not in topological order at task %ld", cu, id);
      last_stage = g.stage_of[id];
    }
  }
  for (int i = 0; i < nt; ++i)
    if (!seen[i]) return fmt("task %ld never queued", i);
  // 3. event counts = number of runs; consumers' thresholds; producers earlier
  std::vector<int> runs(ne, 0), first_prod_stage(ne, 1 << 30), last_prod_stage(ne, -1);
  std::vector<std::vector<int>> prod_in_events(ne);
  for (int cu = 0; cu < c.ncu; ++cu) {
    const auto& q = g.queues[cu];
    for (size_t i = 0; i < q.size(); ++i) {
      const Task& t = g.tasks[q[i]];
      if (t.out_event == kNone16) continue;
      if (t.out_event >= ne) return "task signals an unknown event";
      if (i == 0 || g.tasks[q[i - 1]].out_event != t.out_event) {
        runs[t.out_event]++;
        size_t j = i;
        while (j < q.size() && g.tasks[q[j]].out_event == t.out_event) ++j;
        for (size_t k = i; k < j; ++k)
          if (g.tasks[q[k]].local_count != j - i) return fmt("task %ld: local_count mismatch", q[k]);
      }
      first_prod_stage[t.out_event] = std::min(first_prod_stage[t.out_event], g.stage_of[t.id]);
      last_prod_stage[t.out_event] = std::max(last_prod_stage[t.out_event], g.stage_of[t.id]);
      if (t.in_event != kNone16) prod_in_events[t.out_event].push_back(t.in_event);
    }
  }
  for (int e = 0; e < ne; ++e)
    if ((uint32_t)runs[e] != g.event_count[e]) return fmt("event %ld: count %ld != runs %ld", e, g.event_count[e], runs[e]);
  for (const Task& t : g.tasks) {
    if (t.in_event == kNone16) continue;
    if (t.in_event >= ne) return "task waits on an unknown event";
    if (t.in_count != g.event_count[t.in_event] || t.in_count == 0)
      return fmt("task %ld: threshold %ld != event count %ld", t.id, t.in_count, g.event_count[t.in_event]);
    if (last_prod_stage[t.in_event] >= g.stage_of[t.id])
      return fmt("task %ld waits on an event produced in its own or a later stage", t.id);
  }
  // local slots: runs sharing a slot on one CU are >= kLocalSlots runs apart by construction;
  // also require more than kWorkers tasks between them so that no two are live at once.
  for (int cu = 0; cu < c.ncu; ++cu) {
    std::map<int, int> last_pos;  // slot -> index of the last task of the previous run using it
    const auto& q = g.queues[cu];
    for (size_t i = 0; i < q.size(); ++i) {
      const Task& t = g.tasks[q[i]];
      if (i > 0 && g.tasks[q[i - 1]].out_event == t.out_event) { last_pos[t.local_slot] = (int)i; continue; }
      auto it = last_pos.find(t.local_slot);
      if (it != last_pos.end() && (int)i - it->second <= kWorkers)
        return fmt("CU %ld: local slot %ld reused within %ld tasks", cu, t.local_slot, kWorkers);
      last_pos[t.local_slot] = (int)i;
    }
  }
  // event-level ancestor closure (events are numbered in creation order but
  // compute the closure generically by fixed-point iteration)
  const int words = (ne + 63) / 64;
  std::vector<std::vector<uint64_t>> clo(ne, std::vector<uint64_t>(words, 0));
  for (int e = 0; e < ne; ++e) clo[e][e / 64] |= 1ull << (e % 64);
  for (bool changed = true; changed;) {
    changed = false;
    for (int e = 0; e < ne; ++e)
      for (int pe : prod_in_events[e])
        for (int w = 0; w < words; ++w) {
          uint64_t nv = clo[e][w] | clo[pe][w];
          if (nv != clo[e][w]) { clo[e][w] = nv; changed = true; }
        }
  }
  auto waits_for = [&](int reader_in_ev, int writer_out_ev) -> bool {
    if (reader_in_ev == kNone16 || writer_out_ev == kNone16) return false;
    return ((clo[reader_in_ev][writer_out_ev / 64] >> (writer_out_ev % 64)) & 1) != 0;
  };
  // 4. writes: no overlap (except accumulated buffers); reads covered by ancestors
  std::map<Key, std::vector<Write>> writes;
  std::vector<Region> rd, wr;
  for (const Task& t : g.tasks) {
    task_regions(g, t, rd, wr);
    for (auto& r : wr) writes[key_of(r)].push_back({r.lo, r.hi, (int)t.id});
    if (t.type == TT_QKV && t.a0 < 2) {
      const int half = c.hd / 2, off = t.a1 % c.hd;
      if (t.a3 != half || off >= half || t.a2 != 2) return fmt("task %ld: RoPE pair split across tasks", t.id);
    }
  }
  for (auto& kv : writes) {
    auto& v = kv.second;
    std::sort(v.begin(), v.end(), [](const Write& a, const Write& b) { return a.lo < b.lo || (a.lo == b.lo && a.hi < b.hi); });
    if (std::get<0>(kv.first) == B_LM) continue;
    for (size_t i = 1; i < v.size(); ++i)
      if (v[i].lo < v[i - 1].hi) return fmt("tasks %ld and %ld write the same element", v[i - 1].task, v[i].task);
  }
  // Each output buffer must be written completely.
  auto full_extent = [&](int buf) -> int {
    switch (buf) {
      case B_Q: return c.nq * c.hd;
      case B_K: case B_V: return c.nkv * c.hd;
      case B_PART: return g.nsplit;
      case B_AOUT: return c.nq * c.hd;
      case B_XMID: case B_X: return c.H;
      case B_H: return c.F;
      default: return -1;
    }
  };
  for (auto& kv : writes) {
    const int ext = full_extent(std::get<0>(kv.first));
    if (ext < 0) continue;
    int covered = 0;
    for (auto& w : kv.second) covered += w.hi - w.lo;
    if (covered != ext) return fmt("buffer %ld layer %ld: %ld of %ld elements written", std::get<0>(kv.first), std::get<1>(kv.first), covered, ext);
  }
  std::map<std::tuple<int, int, int, int, int, int>, bool> memo;  // (in_ev, key..., lo, hi)
  for (const Task& t : g.tasks) {
    task_regions(g, t, rd, wr);
    for (auto& r : rd) {
      auto mk = std::make_tuple((int)t.in_event, r.buf * 100000 + r.l, r.b * 4096 + r.grp, r.lo, r.hi, 0);
      auto m = memo.find(mk);
      if (m != memo.end()) {
        if (!m->second) return fmt("task %ld reads data it does not wait for", t.id);
        continue;
      }
      auto it = writes.find(key_of(r));
      if (it == writes.end()) return fmt("task %ld reads a buffer nobody writes (buf %ld)", t.id, r.buf);
      const auto& v = it->second;
      bool ok = true;
      int cur = r.lo;
      // first write whose hi > lo
      auto w = std::lower_bound(v.begin(), v.end(), r.lo, [](const Write& a, int x) { return a.hi <= x; });
      if (r.buf == B_LM) {
        for (auto& ww : v) ok = ok && waits_for(t.in_event, g.tasks[ww.task].out_event);
        cur = r.hi;
      } else {
        for (; w != v.end() && w->lo < r.hi; ++w) {
          if (w->lo > cur) { ok = false; break; }  // gap: element never written
          ok = ok && waits_for(t.in_event, g.tasks[w->task].out_event);
          cur = std::max(cur, w->hi);
        }
      }
      ok = ok && cur >= r.hi;
      memo[mk] = ok;
      if (!ok) return fmt("task %ld reads data it does not wait for (buf %ld layer %ld)", t.id, r.buf, r.l);
    }
  }
  return "";
}

// ---------------------------------------------------------------------------
// Protocol simulator
SimResult simulate_graph(const Graph& g, uint64_t seed, int workers, int drop_event) {
  SimResult res;
  const auto& c = g.cfg;
  const int nt = (int)g.tasks.size();
  std::mt19937_64 rng(seed);
  // Completion counters per written buffer key, and totals.
  std::map<Key, int> need, done;
  std::vector<std::vector<Key>> reads_of(nt), writes_of(nt);
  std::vector<Region> rd, wr;
  for (const Task& t : g.tasks) {
    task_regions(g, t, rd, wr);
    for (auto& r : wr) { need[key_of(r)]++; writes_of[t.id].push_back(key_of(r)); }
    for (auto& r : rd) reads_of[t.id].push_back(key_of(r));
  }
  auto ready_key = [&](const Key& k) { return done[k] == need[k]; };
  std::vector<uint32_t> events(g.event_count.size(), 0);
  struct CuState {
    int frontier = 0, ticket = 0;
    uint16_t cur_key[2] = {0, 0};
    int uses[2] = {0, 0}, page_done[2] = {0, 0};
    std::vector<int> slot = std::vector<int>(kLocalSlots, 0);
    std::vector<int> hold;  // per worker: -1 idle, else ticket
  };
  std::vector<CuState> cus(c.ncu);
  for (auto& s : cus) s.hold.assign(workers, -1);
  bool dropped = false;
  // staged input of a key reads: SK_ATTN_NORM(l>0) X(l); SK_O_IN AOUT(l); SK_FFN_NORM XMID(l); SK_H H(l); FINAL X(L)
  auto stage_reads = [&](uint16_t key, int b) -> Key {
    const int kind = stage_kind(key), l = stage_layer(key);
    switch (kind) {
      case SK_ATTN_NORM: return Key(B_X, l, b, 0);
      case SK_O_IN: return Key(B_AOUT, l, b, 0);
      case SK_FFN_NORM: return Key(B_XMID, l, b, 0);
      case SK_H: return Key(B_H, l, b, 0);
      default: return Key(B_X, c.L, b, 0);
    }
  };
  struct Actor { int cu, w; };  // w == -1: scheduler
  std::vector<Actor> actors;
  for (int cu = 0; cu < c.ncu; ++cu)
    for (int w = -1; w < workers; ++w) actors.push_back({cu, w});
  int executed = 0;
  while (executed < nt) {
    std::shuffle(actors.begin(), actors.end(), rng);
    bool progress = false;
    for (const Actor& a : actors) {
      CuState& s = cus[a.cu];
      const auto& q = g.queues[a.cu];
      const int n = (int)q.size();
      if (a.w < 0) {
        if (s.frontier >= n) continue;
        const Task& t = g.tasks[q[s.frontier]];
        if (t.in_event != kNone16 && events[t.in_event] < t.in_count) continue;
        if (t.stage && s.cur_key[t.page] != t.stage) {
          if (s.page_done[t.page] < s.uses[t.page]) continue;
          if (!(stage_kind(t.stage) == SK_ATTN_NORM && stage_layer(t.stage) == 0)) {
            if (!ready_key(stage_reads(t.stage, t.batch))) {
              res.error = fmt("CU %ld stages input for task %ld before its producers finished", a.cu, t.id);
              return res;
            }
          }
          s.cur_key[t.page] = t.stage;
        }
        if (t.stage) s.uses[t.page]++;
        s.frontier++;
        progress = true;
      } else {
        int& h = s.hold[a.w];
        if (h < 0) {
          if (s.ticket >= n) continue;
          h = s.ticket++;
          progress = true;
          continue;
        }
        if (s.frontier <= h) continue;
        const Task& t = g.tasks[q[h]];
        for (auto& k : reads_of[t.id]) {
          if (std::get<0>(k) == B_X && std::get<1>(k) == 0) continue;
          if (t.stage && k == stage_reads(t.stage, t.batch)) continue;  // read through the page
          if (!ready_key(k)) {
            res.error = fmt("task %ld ran before the data it reads was complete", t.id);
            return res;
          }
        }
        if (t.stage && s.cur_key[t.page] != t.stage) {
          res.error = fmt("task %ld found its LDS page overwritten", t.id);
          return res;
        }
        for (auto& k : writes_of[t.id]) done[k]++;
        if (t.stage) s.page_done[t.page]++;
        if (t.out_event != kNone16) {
          if (++s.slot[t.local_slot] == t.local_count) {
            s.slot[t.local_slot] = 0;
            if (t.out_event == drop_event && !dropped) dropped = true;
            else events[t.out_event]++;
          }
        }
        h = -1;
        ++executed;
        progress = true;
      }
    }
    if (!progress) {
      for (int cu = 0; cu < c.ncu; ++cu) {
        const auto& q = g.queues[cu];
        if (cus[cu].frontier < (int)q.size()) {
          res.blocked_event = g.tasks[q[cus[cu].frontier]].in_event;
          break;
        }
      }
      res.executed = executed;
      return res;
    }
  }
  res.completed = true;
  res.executed = executed;
  return res;
}

// ---------------------------------------------------------------------------
// Batched decode step: stages of tasks
namespace {

const int kBTypes[5] = {TT_QKV, TT_O, TT_GU, TT_DOWN, TT_LM};

bool bad_gemm(const BGemm& m) {
  return m.groups < 1 || m.per_block < 1 || m.blocks < 1 || m.splits < 1 || m.chunk_cols < 1 || m.K < 1 || m.N < 1 ||
         (int64_t)m.blocks * m.per_block < m.groups || (int64_t)(m.blocks - 1) * m.per_block >= m.groups;
}
int gemm_chunks(const BGemm& m) { return (m.K + m.chunk_cols - 1) / m.chunk_cols; }
int gemm_chunks_per_split(const BGemm& m) { return (gemm_chunks(m) + m.splits - 1) / m.splits; }

}  // namespace

std::string build_batched_graph(const BatchedConfig& c, BatchedGraph& g) {
  if (c.B < 2) return "batched graph: B must be >= 2";
  if (c.L < 1 || c.H < 8 || c.nq < 1 || c.nkv < 1 || c.F < 8 || c.V < 1 || c.nsplit < 1)
    return "batched graph: non-positive dimension";
  if (c.nq % c.nkv) return "batched graph: n_q_heads must be a multiple of n_kv_heads";
  for (int t : kBTypes)
    if (bad_gemm(c.gemm[t])) return fmt("batched graph: inconsistent tiling of operator %ld", t);
  if (c.gemm[TT_LM].splits != 1) return "batched graph: the LM head is not split (its argmax runs in the epilogue)";
  g = BatchedGraph();
  g.cfg = c;
  auto stage = [&](uint8_t kind, int type, int layer, int sub, int gx, int gy) {
    g.stages.push_back(BStage{kind, (uint8_t)type, layer, sub, (int)g.tasks.size(), 0, gx, gy});
  };
  auto task = [&](uint8_t kind, int type, int layer, int b, int a0, int a1) {
    g.tasks.push_back(BTask{(int)g.stages.size() - 1, kind, (uint8_t)type, layer, b, a0, a1});
    g.stages.back().count++;
  };
  auto norm = [&](int layer, int kind) {
    stage(BK_NORM, 0, layer, kind, c.B, 1);
    for (int b = 0; b < c.B; ++b) task(BK_NORM, 0, layer, b, kind, 0);
  };
  auto gemm = [&](int type, int layer) {
    const BGemm& m = c.gemm[type];
    stage(BK_GEMM, type, layer, 0, m.blocks, m.splits);
    for (int kz = 0; kz < m.splits; ++kz)
      for (int bx = 0; bx < m.blocks; ++bx) task(BK_GEMM, type, layer, -1, bx, kz);
    if (m.splits > 1) {
      stage(BK_FIN, type, layer, 0, m.groups, 1);
      for (int gr = 0; gr < m.groups; ++gr) task(BK_FIN, type, layer, -1, gr, 0);
    }
  };
  for (int l = 0; l < c.L; ++l) {
    norm(l, 0);
    gemm(TT_QKV, l);
    if (c.nsplit == 1) {
      stage(BK_ATTN_FULL, 0, l, 0, c.B * c.nkv, 1);
      for (int b = 0; b < c.B; ++b)
        for (int grp = 0; grp < c.nkv; ++grp) task(BK_ATTN_FULL, 0, l, b, grp, 0);
    } else {
      stage(BK_ATTN, 0, l, 0, c.B * c.nkv * c.nsplit, 1);
      for (int b = 0; b < c.B; ++b)
        for (int grp = 0; grp < c.nkv; ++grp)
          for (int sp = 0; sp < c.nsplit; ++sp) task(BK_ATTN, 0, l, b, grp, sp);
      // fused: the last split workgroup of each (sequence, KV head) merges inside the attention launch
      stage(BK_MERGE, 0, l, 0, c.fused_merge ? 0 : c.B * c.nkv, c.fused_merge ? 0 : 1);
      for (int b = 0; b < c.B; ++b)
        for (int grp = 0; grp < c.nkv; ++grp) task(BK_MERGE, 0, l, b, grp, 0);
    }
    gemm(TT_O, l);
    norm(l, 1);
    gemm(TT_GU, l);
    gemm(TT_DOWN, l);
  }
  norm(c.L, 2);
  gemm(TT_LM, c.L);
  stage(BK_ARGMAX, 0, c.L, 0, 1, 1);
  task(BK_ARGMAX, 0, c.L, -1, 0, 0);
  return "";
}

namespace {

enum BBuf { BB_XN, BB_Q, BB_K, BB_V, BB_REC, BB_AO, BB_XMID, BB_H, BB_X, BB_PART, BB_COV, BB_KEY, BB_OUT };
struct BRegion {
  int buf, l, b, sub, lo, hi;
};
using BKey = std::tuple<int, int, int, int>;

// Output rows of row group gr of a batched projection (one or two ranges of
// the operator's output buffer), clipped to the matrix.
void group_rows(const BatchedConfig& c, int type, int gr, int& buf, int (&lo)[2], int (&hi)[2], int& n) {
  n = 1;
  switch (type) {
    case TT_QKV: {
      const int per_head = c.hd / 32, nqg = c.nq * per_head, nkg = c.nkv * per_head;
      if (gr < nqg + nkg) {
        const bool isq = gr < nqg;
        const int gg = isq ? gr : gr - nqg, head = gg / per_head, i0 = (gg % per_head) * 16;
        buf = isq ? BB_Q : BB_K;
        lo[0] = head * c.hd + i0;
        lo[1] = head * c.hd + c.hd / 2 + i0;
        hi[0] = lo[0] + 16;
        hi[1] = lo[1] + 16;
        n = 2;
      } else {
        buf = BB_V;
        lo[0] = (gr - nqg - nkg) * 32;
        hi[0] = std::min(lo[0] + 32, c.nkv * c.hd);
      }
      return;
    }
    case TT_O: buf = BB_XMID; lo[0] = gr * 32; hi[0] = std::min(lo[0] + 32, c.H); return;
    case TT_GU: buf = BB_H; lo[0] = gr * 16; hi[0] = std::min(lo[0] + 16, c.F); return;
    case TT_DOWN: buf = BB_X; lo[0] = gr * 32; hi[0] = std::min(lo[0] + 32, c.H); return;
    default: buf = BB_KEY; lo[0] = 0; hi[0] = 1; return;
  }
}

void btask_regions(const BatchedGraph& g, const BTask& t, std::vector<BRegion>& rd, std::vector<BRegion>& wr) {
  const auto& c = g.cfg;
  const int G = c.nq / c.nkv, l = t.layer;
  rd.clear();
  wr.clear();
  // epilogue of row group gr for every sequence: outputs, and the residual
  // rows O and down add (layer 0's O residual is the embedding row)
  auto outputs = [&](int type, int gr) {
    int buf, lo[2], hi[2], n;
    group_rows(c, type, gr, buf, lo, hi, n);
    const int lo_l = type == TT_DOWN ? l + 1 : type == TT_LM ? 0 : l;
    for (int b = 0; b < c.B; ++b)
      for (int i = 0; i < n; ++i) {
        if (lo[i] >= hi[i]) continue;
        wr.push_back({buf, lo_l, b, 0, lo[i], hi[i]});
        if (type == TT_O && l > 0) rd.push_back({BB_X, l, b, 0, lo[i], hi[i]});
        if (type == TT_DOWN) rd.push_back({BB_XMID, l, b, 0, lo[i], hi[i]});
      }
  };
  switch (t.kind) {
    case BK_NORM: {
      const int kind = t.a0;
      if (kind == 0 && l > 0) rd.push_back({BB_X, l, t.b, 0, 0, c.H});
      if (kind == 1) rd.push_back({BB_XMID, l, t.b, 0, 0, c.H});
      if (kind == 2) rd.push_back({BB_X, c.L, t.b, 0, 0, c.H});
      wr.push_back({BB_XN, l, t.b, kind, 0, c.H});
      break;
    }
    case BK_GEMM: {
      const BGemm& m = c.gemm[t.type];
      const int nch = gemm_chunks(m), cps = gemm_chunks_per_split(m);
      const int g0 = t.a0 * m.per_block, g1 = std::min(g0 + m.per_block, m.groups);
      const int c0 = std::min(t.a1 * cps, nch), c1 = std::min(c0 + cps, nch);
      const int k0 = c0 * m.chunk_cols, k1 = std::min(c1 * m.chunk_cols, m.K);
      for (int b = 0; b < c.B; ++b) {
        if (k0 >= k1) break;
        if (t.type == TT_O) rd.push_back({BB_AO, l, b, 0, k0, k1});
        else if (t.type == TT_DOWN) rd.push_back({BB_H, l, b, 0, k0, k1});
        else rd.push_back({BB_XN, l, b, t.type == TT_GU ? 1 : t.type == TT_LM ? 2 : 0, k0, k1});
      }
      const int key = l * 16 + t.type;
      for (int gr = g0; gr < g1; ++gr)
        if (c0 < c1) wr.push_back({BB_COV, key, 0, 0, gr * nch + c0, gr * nch + c1});
      if (m.splits == 1) {
        for (int gr = g0; gr < g1; ++gr) outputs(t.type, gr);
      } else if (g0 < g1) {
        wr.push_back({BB_PART, key, 0, t.a1, g0, g1});
      }
      break;
    }
    case BK_FIN: {
      const BGemm& m = c.gemm[t.type];
      for (int kz = 0; kz < m.splits; ++kz) rd.push_back({BB_PART, l * 16 + t.type, 0, kz, t.a0, t.a0 + 1});
      outputs(t.type, t.a0);
      break;
    }
    case BK_ATTN:
    case BK_ATTN_FULL:
      rd.push_back({BB_Q, l, t.b, 0, t.a0 * G * c.hd, (t.a0 + 1) * G * c.hd});
      rd.push_back({BB_K, l, t.b, 0, t.a0 * c.hd, (t.a0 + 1) * c.hd});
      rd.push_back({BB_V, l, t.b, 0, t.a0 * c.hd, (t.a0 + 1) * c.hd});
      if (t.kind == BK_ATTN) wr.push_back({BB_REC, l, t.b, t.a0, t.a1, t.a1 + 1});
      else wr.push_back({BB_AO, l, t.b, 0, t.a0 * G * c.hd, (t.a0 + 1) * G * c.hd});
      break;
    case BK_MERGE:
      rd.push_back({BB_REC, l, t.b, t.a0, 0, c.nsplit});
      wr.push_back({BB_AO, l, t.b, 0, t.a0 * G * c.hd, (t.a0 + 1) * G * c.hd});
      break;
    case BK_ARGMAX:
      for (int b = 0; b < c.B; ++b) rd.push_back({BB_KEY, 0, b, 0, 0, 1});
      wr.push_back({BB_OUT, 0, 0, 0, 0, c.B});
      break;
  }
}

}  // namespace

std::string validate_batched_graph(const BatchedGraph& g) {
  const auto& c = g.cfg;
  const int ns = (int)g.stages.size(), nt = (int)g.tasks.size();
  // stages partition the tasks in order, and each launch grid holds its tasks
  int next = 0;
  for (int s = 0; s < ns; ++s) {
    const BStage& st = g.stages[s];
    if (st.first != next || st.count < 1) return fmt("stage %ld does not follow its predecessor", s);
    next += st.count;
    for (int i = st.first; i < st.first + st.count; ++i)
      if (g.tasks[i].stage != s || g.tasks[i].kind != st.kind) return fmt("task %ld is not in stage %ld", i, s);
    if (st.gx == 0) {  // merged inside the attention launch before it
      if (st.kind != BK_MERGE || !c.fused_merge || s == 0 || g.stages[s - 1].kind != BK_ATTN)
        return fmt("stage %ld has no launch of its own", s);
    } else if ((int64_t)st.gx * st.gy != st.count) {
      return fmt("stage %ld: grid %ld does not hold its %ld tasks", s, (long)st.gx * st.gy, st.count);
    }
  }
  if (next != nt) return "tasks outside every stage";
  // writes, keyed by buffer; element ranges of one key must not overlap
  struct W { int lo, hi, stage; };
  std::map<BKey, std::vector<W>> writes;
  std::vector<BRegion> rd, wr;
  for (const BTask& t : g.tasks) {
    btask_regions(g, t, rd, wr);
    for (auto& r : wr) writes[BKey(r.buf, r.l, r.b, r.sub)].push_back({r.lo, r.hi, t.stage});
  }
  for (auto& kv : writes) {
    auto& v = kv.second;
    std::sort(v.begin(), v.end(), [](const W& a, const W& b) { return a.lo < b.lo || (a.lo == b.lo && a.hi < b.hi); });
    if (std::get<0>(kv.first) == BB_KEY) continue;  // a maximum over many writers
    for (size_t i = 1; i < v.size(); ++i)
      if (v[i].lo < v[i - 1].hi)
        return fmt("buffer %ld (layer key %ld): element %ld written twice", std::get<0>(kv.first), std::get<1>(kv.first),
                   v[i].lo);
  }
  // every written buffer complete (per sequence, per layer)
  auto extent = [&](const BKey& k) -> int64_t {
    const int buf = std::get<0>(k);
    switch (buf) {
      case BB_XN: case BB_XMID: case BB_X: return c.H;
      case BB_Q: case BB_AO: return (int64_t)c.nq * c.hd;
      case BB_K: case BB_V: return (int64_t)c.nkv * c.hd;
      case BB_REC: return c.nsplit;
      case BB_H: return c.F;
      case BB_OUT: return c.B;
      case BB_PART: return c.gemm[std::get<1>(k) % 16].groups;
      case BB_COV: {
        const BGemm& m = c.gemm[std::get<1>(k) % 16];
        return (int64_t)m.groups * gemm_chunks(m);
      }
      default: return -1;
    }
  };
  for (auto& kv : writes) {
    const int64_t ext = extent(kv.first);
    if (ext < 0) continue;
    int64_t covered = 0;
    for (auto& w : kv.second) covered += w.hi - w.lo;
    if (covered != ext)
      return fmt("buffer %ld (layer key %ld): %ld of %ld elements written", std::get<0>(kv.first),
                 std::get<1>(kv.first), covered, ext);
  }
  // each sequence's every buffer of every layer exists
  for (int l = 0; l < c.L; ++l)
    for (int b = 0; b < c.B; ++b)
      for (int buf : {BB_Q, BB_K, BB_V, BB_AO, BB_XMID, BB_H, BB_X})
        if (!writes.count(BKey(buf, buf == BB_X ? l + 1 : l, b, 0)))
          return fmt("layer %ld sequence %ld: buffer %ld never written", l, b, buf);
  // reads: covered by writes of earlier stages
  for (const BTask& t : g.tasks) {
    btask_regions(g, t, rd, wr);
    for (auto& r : rd) {
      auto it = writes.find(BKey(r.buf, r.l, r.b, r.sub));
      if (it == writes.end()) return fmt("task %ld reads a buffer nobody writes (buf %ld)", (long)(&t - &g.tasks[0]), r.buf);
      int cur = r.lo;
      for (const W& w : it->second) {
        if (w.hi <= cur) continue;
        if (w.lo >= r.hi) break;
        if (w.lo > cur) break;  // gap
        if (w.stage >= t.stage)
          return fmt("task %ld reads buffer %ld written by stage %ld, not before it", (long)(&t - &g.tasks[0]), r.buf,
                     w.stage);
        cur = std::max(cur, w.hi);
        if (cur >= r.hi) break;
      }
      if (r.buf != BB_KEY && cur < r.hi)
        return fmt("task %ld reads elements [%ld, %ld) of buffer %ld that no task writes", (long)(&t - &g.tasks[0]), cur,
                   r.hi, r.buf);
    }
  }
  return "";
}

int64_t batched_weight_bytes(const BatchedGraph& g) {
  const auto& c = g.cfg;
  int64_t bytes = 0;
  for (const BTask& t : g.tasks) {
    if (t.kind != BK_GEMM) continue;
    const BGemm& m = c.gemm[t.type];
    const int nch = gemm_chunks(m), cps = gemm_chunks_per_split(m);
    const int c0 = std::min(t.a1 * cps, nch), c1 = std::min(c0 + cps, nch);
    const int64_t cols = std::max(0, std::min(c1 * m.chunk_cols, m.K) - c0 * m.chunk_cols);
    const int g0 = t.a0 * m.per_block, g1 = std::min(g0 + m.per_block, m.groups);
    for (int gr = g0; gr < g1; ++gr) {
      int buf, lo[2], hi[2], n;
      if (t.type == TT_LM) {
        lo[0] = gr * 32; hi[0] = std::min(lo[0] + 32, c.V); n = 1;
      } else {
        group_rows(c, t.type, gr, buf, lo, hi, n);
      }
      int64_t rows = 0;
      for (int i = 0; i < n; ++i) rows += std::max(0, hi[i] - lo[i]);
      bytes += rows * cols * 2 * (t.type == TT_GU ? 2 : 1);
    }
  }
  return bytes;
}

}  // namespace mk
