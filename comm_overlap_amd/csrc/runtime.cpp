// Slice scheduler and C-ABI entry points of the sliced layer shard.
//
// Every call forks from the caller's stream onto the plan's worker streams, runs row slice i on
// worker i mod S (its products in order), records an event after each finished hand-off piece and
// lets a copy stream wait on that event and move the piece with a DMA-engine copy while the
// workers go on computing - the single-GPU stand-in for handing the piece to the tensor-parallel
// reduction (Domino page, Abstract: independent pieces whose communication overlaps later
// computation; FiCCO page, Abstract: communication offloaded to the GPU's DMA engines; DHelix
// review, Referee report: separate computation and communication streams joined by barriers).
// At the end the caller's stream waits on every worker and copy stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "attn.hpp"
#include "gemm.hpp"
#include "plan.hpp"

namespace tps {
static_assert(kColsumChunkRows == kColsumRows, "workspace sizing and the column-sum kernel disagree");
namespace {

struct TraceSlot {
  tpslice_trace_rec_t rec;
  size_t ev0, ev1;  // indices into Runtime::tpool
};

struct Runtime {
  int device = -1;
  // worker 0 is the caller's stream (TPSLICE_F_CALLER_WORKER): the caller passes S - 1 worker
  // streams, else S
  int32_t first_own_worker = 0;
  hipEvent_t fork = nullptr;
  // end of the latest call on its caller's stream (TPSLICE_F_CALLER_WORKER: a call from another
  // stream waits for it, since the plan's workspace and worker 0 went with the previous caller)
  hipEvent_t call_done = nullptr;
  hipStream_t last_caller = nullptr;
  bool have_last = false;
  // the latest call queued products over all tokens after its last hand-off (weight gradients,
  // the QKV projection): its copies ran under them, so the next call's first row slice can wait
  // for all of them at once, at no cost, instead of each row slice for its own
  bool tail_after_copies = false;
  std::vector<hipEvent_t> piece;   // one per hand-off piece (and reused per call)
  std::vector<hipEvent_t> lead;    // one per row slice: its first product is done
  std::vector<hipEvent_t> gather;  // one per worker stream: its queued products are done
  std::vector<hipEvent_t> join_w, join_c;
  // pipelined hand-off: per (row slice, copy stream) completion of the latest call's copies
  std::vector<hipEvent_t> copied;       // [r][E]
  std::vector<uint8_t> copied_pending;  // [r][E]: recorded and not yet superseded
  // Order of the records of `copied`: copied_seq[x] numbers the latest record of event x, and
  // copied_on[x] names the (copy stream, call) it was recorded in. A stream completes its work in
  // order, so a wait for one record covers every earlier record that the same call queued on the
  // same stream (records of different calls are not compared: the caller may pass other streams).
  // covered[w]: per (stream, call), the latest record that worker stream w has waited for in the
  // current call (cleared at each call's start).
  struct CopyKey {
    hipStream_t stream;
    uint64_t call;
    bool operator==(const CopyKey& o) const { return stream == o.stream && call == o.call; }
  };
  uint64_t copy_seq = 0, call_serial = 0;
  std::vector<uint64_t> copied_seq;
  std::vector<CopyKey> copied_on;
  std::vector<std::vector<std::pair<CopyKey, uint64_t>>> covered;
  // tracing: timing events, recorded around each product / copy of the latest call
  hipEvent_t t0 = nullptr;
  bool window_open = false;
  int32_t calls = 0;
  std::vector<hipEvent_t> tpool;
  size_t tused = 0;
  std::vector<TraceSlot> slots;
};

#define TPS_TRY_(x)                    \
  do {                                 \
    tpslice_status_t st_ = (x);        \
    if (st_ != TPSLICE_OK) return st_; \
  } while (0)

#define TPS_HIP(call)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess) return fail(TPSLICE_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// Every event is waited for before it is destroyed, so no queued work - on the caller's stream (a
// one-worker plan's products, the join), a worker or a copy stream - still records or waits on
// it. The streams belong to the caller and are left alone.
void drop_event(hipEvent_t& e) {
  if (!e) return;
  (void)hipEventSynchronize(e);
  (void)hipEventDestroy(e);
  e = nullptr;
}

void destroy_runtime(Runtime* rt) {
  if (!rt) return;
  drop_event(rt->fork);
  drop_event(rt->call_done);
  for (auto* v : {&rt->piece, &rt->lead, &rt->gather, &rt->join_w, &rt->join_c, &rt->copied, &rt->tpool})
    for (auto& e : *v) drop_event(e);
  drop_event(rt->t0);
  delete rt;
}

// Events that order products on worker streams against each other and against the caller's stream
// (`local`) skip the system-scope fence of their release and acquire: the products and their
// consumers are kernels on this GPU, ordered at device scope. Events in front of a DMA-engine copy
// and after one keep the system-scope fence. Measured on the same GPU in alternation: Llama-2 13B
// layer 732 -> 750 TFLOP/s, Llama-2 7B MLP 931 -> 954; with every event local, the 7B MLP varied
// 914-959 and hid less of its copy time.
tpslice_status_t make_event(hipEvent_t* e, bool local = false) {
  TPS_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming | (local ? hipEventDisableSystemFence : 0u)));
  return TPSLICE_OK;
}

// The plan's events are created on its first call, on the device current at that time. A failure
// part way leaves no runtime behind (the next call starts over).
tpslice_status_t build_runtime(tpslice_plan_s* p, Runtime* rt) {
  if (p->desc.flags & TPSLICE_F_SERIALIZE) return TPSLICE_OK;  // one stream, no events
  rt->first_own_worker = (p->desc.flags & TPSLICE_F_CALLER_WORKER) ? 1 : 0;
  rt->join_w.assign(p->S, nullptr);
  rt->join_c.assign(p->E, nullptr);
  rt->piece.assign(size_t(p->r) * p->c, nullptr);
  rt->lead.assign(p->r, nullptr);
  rt->gather.assign(p->S, nullptr);
  rt->copied.assign(size_t(p->r) * p->E, nullptr);
  rt->copied_pending.assign(size_t(p->r) * p->E, 0);
  rt->copied_seq.assign(size_t(p->r) * p->E, 0);
  rt->copied_on.assign(size_t(p->r) * p->E, Runtime::CopyKey{nullptr, 0});
  rt->covered.assign(size_t(p->S), {});
  for (auto& c : rt->covered) c.reserve(size_t(kMaxCopyStreams) * 2);
  TPS_TRY_(make_event(&rt->fork, true));
  TPS_TRY_(make_event(&rt->call_done, true));
  for (auto& e : rt->join_w) TPS_TRY_(make_event(&e, true));
  for (auto& e : rt->join_c) TPS_TRY_(make_event(&e));
  // the hand-off events ride on the products' launches (hipExtLaunchKernelGGL's stop event), whose
  // documented use is a timing event: created with timing, and with the system-scope fence that
  // the DMA engine's copy after them needs
  for (auto& e : rt->piece) TPS_HIP(hipEventCreateWithFlags(&e, hipEventDefault));
  // the first-product events ride on launches too (see the hand-off events): with timing, and
  // without the system-scope fence (their consumers are kernels on this GPU)
  for (auto& e : rt->lead) TPS_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  for (auto& e : rt->gather) TPS_TRY_(make_event(&e, true));
  for (auto& e : rt->copied) TPS_TRY_(make_event(&e));
  return TPSLICE_OK;
}

tpslice_status_t ensure_runtime(tpslice_plan_s* p, Runtime** out) {
  int dev = -1;
  TPS_HIP(hipGetDevice(&dev));
  Runtime* rt = static_cast<Runtime*>(p->rt);
  if (rt) {
    if (rt->device != dev)
      return fail(TPSLICE_ERR_UNSUPPORTED, "plan was first used on device %d, now device %d", rt->device, dev);
    *out = rt;
    return TPSLICE_OK;
  }
  rt = new (std::nothrow) Runtime();
  if (!rt) return fail(TPSLICE_ERR_INVALID, "out of host memory");
  rt->device = dev;
  const tpslice_status_t st = build_runtime(p, rt);
  if (st != TPSLICE_OK) {
    destroy_runtime(rt);
    return st;
  }
  p->rt = rt;
  *out = rt;
  return TPSLICE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// One call's stream bookkeeping.
struct Schedule {
  tpslice_plan_s* p;
  Runtime* rt;
  hipStream_t caller;
  bool serial;
  const hipStream_t* own_workers;  // the caller's worker streams (workers first_own_worker..S-1)
  const hipStream_t* copiers;      // the caller's copy streams (E of them), or NULL: no hand-off
  uint32_t copied = 0;  // bit k: copy stream k received a copy in this call (bit 31: caller stream)
  uint32_t slice_streams = 0;  // copy streams used by the current row slice's pieces
  int lead_slice = -1;         // row slice whose first product has not been queued yet
  int lead_done = -1;          // latest row slice whose first-product event this call recorded
  bool attached = false;       // the latest product's launch records its hand-off event itself
  bool tail = false;           // a product over all tokens follows this call's latest hand-off
  bool eager = false;          // the first row slice waits for every pending copy of earlier calls
  bool capturing = false;      // the caller's stream is capturing a graph: events are recorded by
                               // markers (an event bound to a captured launch orders nothing)

  tpslice_status_t fence(hipStream_t s) {
    hipError_t e = launch_fence(s);
    if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "fence launch: %s", hipGetErrorString(e));
    return TPSLICE_OK;
  }

  // worker stream k: the caller's stream when serialized, or for k = 0 with TPSLICE_F_CALLER_WORKER
  hipStream_t wk(int k) const {
    return serial || k < rt->first_own_worker ? caller : own_workers[k - rt->first_own_worker];
  }
  hipStream_t cp(int k) const { return copiers[k]; }
  hipStream_t worker(int i) const { return wk(i % p->S); }
  int worker_id(int i) const { return serial ? -1 : i % p->S; }
  bool pipelined() const { return !serial && (p->desc.flags & TPSLICE_F_PIPELINE); }

  // Row slices on different worker streams start in order: slice i's first product waits for
  // slice i-1's first product, so it runs beside slice i-1's later products (filling the compute
  // units they leave idle) and the slices finish one after another, each hand-off starting while
  // later slices still compute. Pipelined mode: row slice i's products also wait for the previous
  // call's hand-off of row slice i.
  // `span`: row slices i .. i + span - 1 whose rows the slice's first product reads (a product over
  // a group of row slices waits for the previous call's hand-off of each of them).
  tpslice_status_t slice_begin(int i, int span = 1) {
    if (serial) return TPSLICE_OK;
    // the next slice waits for this one's first product only from another worker stream (one
    // worker: stream order already does it, and an event between two products costs their gap)
    lead_slice = i + 1 < p->r && worker(i + 1) != worker(i) ? i : -1;
    if (i > 0 && lead_done == i - 1 && worker(i) != worker(i - 1))
      TPS_HIP(hipStreamWaitEvent(worker(i), rt->lead[i - 1], 0));
    if (!pipelined()) return TPSLICE_OK;
    if (eager) {
      eager = false;
      return wait_copies(i % p->S, 0, p->r);
    }
    return wait_copies(i % p->S, i, std::min(i + span, p->r));
  }

  // Worker stream w waits for the pending copies of row slices [q0, q1): on each copy stream, one
  // wait for the latest of their records that w has not yet covered in this call (each wait costs
  // the gap between two products: a producer over a group of row slices needs one per copy stream,
  // not one per row slice, and the row slices after it none).
  tpslice_status_t wait_copies(int w, int q0, int q1) {
    auto& cov = rt->covered[size_t(w)];
    auto covered_seq = [&](const Runtime::CopyKey& st) -> uint64_t* {
      for (auto& c : cov)
        if (c.first == st) return &c.second;
      return nullptr;
    };
    // one round per stream that holds uncovered records of the range (normally one per copy
    // stream): a wait for that stream's latest uncovered record covers all of them
    auto uncovered = [&](size_t x) {
      if (!rt->copied_pending[x]) return false;
      const uint64_t* c = covered_seq(rt->copied_on[x]);
      return !c || rt->copied_seq[x] > *c;
    };
    const size_t x0 = size_t(q0) * p->E, x1 = size_t(q1) * p->E;
    for (;;) {
      size_t first = SIZE_MAX;
      for (size_t x = x0; x < x1 && first == SIZE_MAX; ++x)
        if (uncovered(x)) first = x;
      if (first == SIZE_MAX) return TPSLICE_OK;
      const Runtime::CopyKey st = rt->copied_on[first];
      size_t best = first;
      for (size_t x = first + 1; x < x1; ++x)
        if (uncovered(x) && rt->copied_on[x] == st && rt->copied_seq[x] > rt->copied_seq[best]) best = x;
      TPS_HIP(hipStreamWaitEvent(wk(w), rt->copied[best], 0));
      if (uint64_t* c = covered_seq(st)) *c = rt->copied_seq[best];
      else cov.emplace_back(st, rt->copied_seq[best]);
    }
  }

  // Pipelined mode: worker k waits for every hand-off copy of the previous calls that has not been
  // waited for, before a product over all tokens that no row slice of this call precedes (it may
  // read rows of every slice of a previous call's hand-off buffer).
  tpslice_status_t wait_all_handoffs(int k) {
    if (!pipelined()) return TPSLICE_OK;
    return wait_copies(k, 0, p->r);
  }

  // Pipelined mode: mark the end of row slice i's hand-off copies on each copy stream it used.
  tpslice_status_t slice_handed_off(int i, uint32_t streams_used) {
    if (!pipelined()) return TPSLICE_OK;
    for (int k = 0; k < p->E; ++k) {
      if (!(streams_used & (1u << k))) continue;
      TPS_TRY_(fence(cp(k)));
      const size_t x = size_t(i) * p->E + k;
      TPS_HIP(hipEventRecord(rt->copied[x], cp(k)));
      rt->copied_pending[x] = 1;
      rt->copied_seq[x] = ++rt->copy_seq;
      rt->copied_on[x] = Runtime::CopyKey{cp(k), rt->call_serial};
    }
    return TPSLICE_OK;
  }

  tpslice_status_t trace_event(size_t* idx) {
    if (rt->tused == rt->tpool.size()) {
      hipEvent_t e;
      TPS_HIP(hipEventCreate(&e));
      rt->tpool.push_back(e);
    }
    *idx = rt->tused++;
    return TPSLICE_OK;
  }

  // Run `fn` (which queues work on `s`) between two timing events when tracing. A traced copy is
  // closed by a fence kernel so that its end event waits for the DMA engine.
  template <class F>
  tpslice_status_t traced(hipStream_t s, int stream_id, int kind, int step, int slice, int piece, double flops,
                          double bytes, F&& fn) {
    if (kind == TPSLICE_TRACE_COPY) {
      const uint32_t bit = stream_id < 0 ? (1u << 31) : (1u << (stream_id - p->S));
      copied |= bit;
      slice_streams |= bit;
    }
    const int32_t want = kind == TPSLICE_TRACE_COPY ? 2 : 1;
    if (!(p->trace & want)) return fn();
    TraceSlot t{};
    t.rec.kind = kind; t.rec.step = step; t.rec.slice = slice; t.rec.piece = piece;
    t.rec.stream = stream_id; t.rec.flops = flops; t.rec.bytes = bytes; t.rec.call = rt->calls - 1;
    TPS_TRY_(trace_event(&t.ev0));
    TPS_HIP(hipEventRecord(rt->tpool[t.ev0], s));
    TPS_TRY_(fn());
    if (kind == TPSLICE_TRACE_COPY) TPS_TRY_(fence(s));
    TPS_TRY_(trace_event(&t.ev1));
    TPS_HIP(hipEventRecord(rt->tpool[t.ev1], s));
    rt->slots.push_back(t);
    return TPSLICE_OK;
  }

  tpslice_status_t fork() {
    for (auto& c : rt->covered) c.clear();
    ++rt->call_serial;
    eager = rt->tail_after_copies;
    if (p->trace) {
      if (!rt->window_open) {
        if (!rt->t0) TPS_HIP(hipEventCreate(&rt->t0));
        TPS_HIP(hipEventRecord(rt->t0, caller));
        rt->window_open = true;
        rt->calls = 0;
      }
      ++rt->calls;
    }
    if (serial) return TPSLICE_OK;
    if (rt->first_own_worker && rt->have_last && rt->last_caller != caller)
      TPS_HIP(hipStreamWaitEvent(caller, rt->call_done, 0));
    // With worker 0 on the caller's stream every copy waits for a piece event recorded on a worker
    // stream that is itself ordered after the caller's earlier work (worker 0 is the caller, the
    // others wait for the fork), so the copy streams need no fork of their own; with no other
    // worker stream there is nothing to fork.
    const bool copier_fork = !rt->first_own_worker && copiers;
    if (rt->first_own_worker >= p->S && !copier_fork) return TPSLICE_OK;
    TPS_HIP(hipEventRecord(rt->fork, caller));
    for (int k = rt->first_own_worker; k < p->S; ++k) TPS_HIP(hipStreamWaitEvent(wk(k), rt->fork, 0));
    if (copier_fork)
      for (int k = 0; k < p->E; ++k) TPS_HIP(hipStreamWaitEvent(cp(k), rt->fork, 0));
    return TPSLICE_OK;
  }

  // The caller's stream waits for every worker and copy stream. DMA-engine copies are closed by a
  // fence kernel first, so that the join event covers their completion.
  tpslice_status_t join() {
    rt->tail_after_copies = tail;
    if (serial) {
      if (copied) TPS_TRY_(fence(caller));
      return TPSLICE_OK;
    }
    for (int k = rt->first_own_worker; k < p->S; ++k) {
      TPS_HIP(hipEventRecord(rt->join_w[k], wk(k)));
      TPS_HIP(hipStreamWaitEvent(caller, rt->join_w[k], 0));
    }
    if (!pipelined() && copiers) {  // (pipelined: hand-off copies are joined per slice by later calls)
      for (int k = 0; k < p->E; ++k) {
        if (copied & (1u << k)) TPS_TRY_(fence(cp(k)));
        TPS_HIP(hipEventRecord(rt->join_c[k], cp(k)));
        TPS_HIP(hipStreamWaitEvent(caller, rt->join_c[k], 0));
      }
    }
    if (rt->first_own_worker) {
      TPS_HIP(hipEventRecord(rt->call_done, caller));
      rt->last_caller = caller;
      rt->have_last = true;
    }
    return TPSLICE_OK;
  }

  // Hand-off of piece (i, j) of a [M][h] bf16 tensor produced on worker(i).
  tpslice_status_t handoff(int i, int j, const void* src, void* dst) {
    const int64_t row0 = int64_t(i) * p->Ms, col0 = int64_t(j) * p->hc;
    const size_t pitch = size_t(p->h) * 2;
    const char* s = static_cast<const char*>(src) + row0 * pitch + col0 * 2;
    char* d = static_cast<char*>(dst) + row0 * pitch + col0 * 2;
    const hipMemcpyKind kind =
        (p->desc.flags & TPSLICE_F_COPY_BLIT) ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToDeviceNoCU;
    // whole row slices: one contiguous copy after the slice's last product (its products then
    // span all columns: p->pc == 1)
    const bool rows = p->c > 1 && (p->desc.flags & TPSLICE_F_HANDOFF_ROWS);
    if (rows) {
      if (j < p->pc - 1) return TPSLICE_OK;
      s = static_cast<const char*>(src) + row0 * pitch;
      d = static_cast<char*>(dst) + row0 * pitch;
    }
    const bool contiguous = p->c == 1 || rows;
    const double piece_bytes = double(p->Ms) * double(contiguous ? p->h : p->hc) * 2.0;
    if (serial) {
      return traced(caller, -1, TPSLICE_TRACE_COPY, TPSLICE_STEP_HANDOFF, i, j, 0.0, piece_bytes, [&] {
        if (contiguous) TPS_HIP(hipMemcpyAsync(d, s, size_t(p->Ms) * pitch, kind, caller));
        else TPS_HIP(hipMemcpy2DAsync(d, pitch, s, pitch, size_t(p->hc) * 2, size_t(p->Ms), kind, caller));
        return TPSLICE_OK;
      });
    }
    hipEvent_t ev = rt->piece[size_t(i) * p->c + j];
    if (!attached) TPS_HIP(hipEventRecord(ev, worker(i)));
    attached = false;
    tail = false;
    if (contiguous) {
      // a whole-row piece is contiguous: spread it over the copy streams in equal row chunks
      const int64_t E = p->E;
      for (int64_t k = 0; k < E; ++k) {
        const int64_t r0 = p->Ms * k / E, r1 = p->Ms * (k + 1) / E;
        if (r1 <= r0) continue;
        hipStream_t cs = cp(k);
        TPS_HIP(hipStreamWaitEvent(cs, ev, 0));
        const size_t nbytes = size_t(r1 - r0) * pitch;
        TPS_TRY_(traced(cs, p->S + int(k), TPSLICE_TRACE_COPY, TPSLICE_STEP_HANDOFF, i, j, 0.0, double(nbytes), [&] {
          TPS_HIP(hipMemcpyAsync(d + r0 * pitch, s + r0 * pitch, nbytes, kind, cs));
          return TPSLICE_OK;
        }));
      }
    } else {
      const int k = int((size_t(i) * p->c + j) % p->E);
      hipStream_t cs = cp(k);
      TPS_HIP(hipStreamWaitEvent(cs, ev, 0));
      TPS_TRY_(traced(cs, p->S + k, TPSLICE_TRACE_COPY, TPSLICE_STEP_HANDOFF, i, j, 0.0, piece_bytes, [&] {
        TPS_HIP(hipMemcpy2DAsync(d, pitch, s, pitch, size_t(p->hc) * 2, size_t(p->Ms), kind, cs));
        return TPSLICE_OK;
      }));
    }
    return TPSLICE_OK;
  }

  // The kernel identity of the latest GEMM launch, for a trace record.
  static void tag_kernel(tpslice_trace_rec_t& rec) {
    const LaunchInfo k = last_launch();
    rec.tile_m = k.bm; rec.tile_n = k.bn; rec.waves_m = k.waves_m; rec.waves_n = k.waves_n;
    rec.blocks_per_cu = k.blocks_per_cu; rec.layout = k.layout; rec.epilogue = k.epi;
    rec.blocks = k.blocks; rec.threads = k.threads;
  }

  // Queue one product on worker(i) (i = -1: worker `on`, all tokens), traced as `step`. A traced
  // product carries its timing events on the dispatch itself.
  // `alone`: nothing else runs beside this product (an all-token product after the slices), so the
  // tile choice may take the tiles that fill the last round
  // A launch may record an ordering event itself (its dispatch's stop event) instead of a marker
  // after it: not when traced (the dispatch carries the timing events), not under graph capture
  // (an event bound to a captured launch orders nothing) and not on the serialized stream.
  bool bind_ok(bool traced) const { return !serial && !traced && !capturing; }

  // After row slice i's first product: the next row slice (on another worker) waits for it.
  tpslice_status_t lead_recorded(int i, bool bound) {
    if (i < 0 || i != lead_slice) return TPSLICE_OK;
    if (!bound) TPS_HIP(hipEventRecord(rt->lead[i], worker(i)));
    lead_slice = -1;
    lead_done = i;
    return TPSLICE_OK;
  }

  // `handoff`: piece (i, piece) of this product is handed off next (handoff()); an untraced launch
  // then records the piece's event itself at the kernel's end, with no marker between this product
  // and the next (a marker costs the gap between two products, about 5 us).
  tpslice_status_t product(int i, int step, int piece, const GemmArgs& g, int layout, int epi, int on = 0,
                           bool alone = false, bool handoff = false) {
    const int wi = i < 0 ? on : i;
    const double flops = 2.0 * double(g.M) * double(g.N) * double(g.K) * (epi == kEpiSwiglu ? 2.0 : 1.0);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    TraceSlot t{};
    const bool tr = (p->trace & 1) && g.M > 0 && g.N > 0;
    if (tr) {
      t.rec.kind = TPSLICE_TRACE_GEMM; t.rec.step = step; t.rec.slice = i; t.rec.piece = piece;
      t.rec.stream = worker_id(wi); t.rec.flops = flops; t.rec.call = rt->calls - 1;
      TPS_TRY_(trace_event(&t.ev0));
      TPS_TRY_(trace_event(&t.ev1));
      e0 = rt->tpool[t.ev0];
      e1 = rt->tpool[t.ev1];
    }
    // the event this launch records at its end: the piece's hand-off event, else the row slice's
    // first-product event that the next row slice (on another worker) waits for
    hipEvent_t done = nullptr;
    bool lead_bound = false;
    if (bind_ok(tr) && i >= 0 && g.M > 0 && g.N > 0) {
      if (handoff) done = rt->piece[size_t(i) * p->c + size_t(piece)];
      else if (i == lead_slice) { done = rt->lead[i]; lead_bound = true; }
    }
    hipError_t e = launch_gemm(g, layout, epi, worker(wi), e0, done ? done : e1, p->tile,
                               alone || serial || p->S == 1);
    if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "GEMM launch: %s", hipGetErrorString(e));
    attached = done != nullptr && !lead_bound;
    if (i < 0) tail = true;
    TPS_TRY_(lead_recorded(i, lead_bound));
    if (tr) {
      tag_kernel(t.rec);
      rt->slots.push_back(t);
    }
    return TPSLICE_OK;
  }

  // A product split along k when `splits` > 1: fp32 partials in `part`, then the ordered
  // reduction with the product's epilogue. i >= 0: row slice i's product (on worker(i));
  // i < 0: a product over all tokens on worker(on). tail_rows > 0: only the product's last
  // tail_rows rows are split, the others run unsplit between the partials and the reduction.
  // Traced as two records: the GEMM of the partial products and of the unsplit rows (with the
  // product's flops) and the reduction.
  tpslice_status_t product_split(int i, int step, int piece, const GemmArgs& g, int layout, int epi, int splits,
                                 float* part, int on = 0, bool alone = false, int64_t tail_rows = 0) {
    if (splits <= 1) return product(i, step, piece, g, layout, epi, on, alone);
    if (i < 0) tail = true;
    const int wi = i < 0 ? on : i;
    const double flops = 2.0 * double(g.M) * double(g.N) * double(g.K) * (epi == kEpiSwiglu ? 2.0 : 1.0);
    hipEvent_t e0 = nullptr, em = nullptr, e1 = nullptr;
    TraceSlot t{}, u{};
    const bool tr = (p->trace & 1) && g.M > 0 && g.N > 0;
    if (tr) {
      t.rec.kind = TPSLICE_TRACE_GEMM; t.rec.step = step; t.rec.slice = i; t.rec.piece = piece;
      t.rec.stream = worker_id(wi); t.rec.flops = flops; t.rec.call = rt->calls - 1;
      u.rec = t.rec;
      u.rec.kind = TPSLICE_TRACE_SPLIT_SUM;
      u.rec.flops = 0.0;
      TPS_TRY_(trace_event(&t.ev0));
      TPS_TRY_(trace_event(&t.ev1));
      TPS_TRY_(trace_event(&u.ev1));
      u.ev0 = t.ev1;
      e0 = rt->tpool[t.ev0];
      em = rt->tpool[t.ev1];
      e1 = rt->tpool[u.ev1];
    }
    const bool lead_bound = bind_ok(tr) && i >= 0 && i == lead_slice && g.M > 0 && g.N > 0;
    if (lead_bound) e1 = rt->lead[i];  // the reduction, the product's last launch, records it
    hipError_t e = launch_gemm_split(g, layout, epi, splits, part, worker(wi), e0, e1, p->tile, em, tail_rows);
    if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "split GEMM launch: %s", hipGetErrorString(e));
    TPS_TRY_(lead_recorded(i, lead_bound));
    if (tr) {
      tag_kernel(t.rec);
      rt->slots.push_back(t);
      rt->slots.push_back(u);
    }
    return TPSLICE_OK;
  }

  // This call's partial buffer of worker(i) for a split per-slice product (regions of `bytes`
  // each from `base`, one per worker stream).
  float* slice_part(char* base, size_t bytes, int i) const {
    return reinterpret_cast<float*>(base + size_t(serial ? 0 : i % p->S) * bytes);
  }

  tpslice_status_t colsum(const void* X, int64_t ld, int64_t M, int64_t N, float* partials, float* out,
                          int accumulate, int on = 0) {
    return traced(worker(on), worker_id(on), TPSLICE_TRACE_COLSUM, TPSLICE_STEP_BIAS_GRAD, -1, -1, 0.0,
                  double(M) * double(N) * 2.0, [&] {
      hipError_t e = launch_colsum(X, ld, int32_t(M), int32_t(N), partials, out, accumulate, worker(on));
      if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "column-sum launch: %s", hipGetErrorString(e));
      return TPSLICE_OK;
    });
  }

  // Make every worker stream wait until every row slice's products are finished, so that the
  // products over all tokens that follow can be spread over the workers.
  tpslice_status_t gather_slices() {
    if (serial || p->S == 1) return TPSLICE_OK;
    for (int k = 0; k < p->S; ++k) TPS_HIP(hipEventRecord(rt->gather[k], wk(k)));
    for (int k = 0; k < p->S; ++k)
      for (int q = 0; q < p->S; ++q)
        if (q != k) TPS_HIP(hipStreamWaitEvent(wk(k), rt->gather[q], 0));
    return TPSLICE_OK;
  }
};

// The caller's streams for one call, checked before anything is queued. With
// TPSLICE_F_CALLER_WORKER worker 0 is the caller's stream and the caller passes S - 1 worker
// streams, else S; a call with hand-off copies also takes E copy streams. The streams one call
// uses must all differ. A serialized plan uses the caller's stream only.
struct CallStreams {
  hipStream_t caller = nullptr;
  bool serial = false;
  hipStream_t workers[kMaxStreams] = {};
  hipStream_t copiers[kMaxCopyStreams] = {};
  bool have_copiers = false;
  bool capturing = false;  // the caller's stream is capturing a HIP graph
};

tpslice_status_t call_streams(const tpslice_plan_s* p, const tpslice_streams_t* s, bool copies, CallStreams* out) {
  out->caller = s ? static_cast<hipStream_t>(s->caller) : nullptr;
  out->serial = p->desc.flags & TPSLICE_F_SERIALIZE;
  if (out->serial) return TPSLICE_OK;
  const int need_w = p->S - ((p->desc.flags & TPSLICE_F_CALLER_WORKER) ? 1 : 0);
  const int need_c = copies ? p->E : 0;
  const int have_w = s ? s->n_workers : 0, have_c = s ? s->n_copiers : 0;
  if (have_w < need_w || (need_w > 0 && !s->workers))
    return fail(TPSLICE_ERR_INVALID, "the plan runs on %d worker stream(s) of the caller's, %d given", need_w,
                have_w);
  if (have_c < need_c || (need_c > 0 && !s->copiers))
    return fail(TPSLICE_ERR_INVALID, "the hand-off needs %d copy stream(s), %d given", need_c, have_c);
  hipStream_t used[1 + kMaxStreams + kMaxCopyStreams];
  int n = 0;
  used[n++] = out->caller;
  for (int k = 0; k < need_w; ++k) used[n++] = out->workers[k] = static_cast<hipStream_t>(s->workers[k]);
  for (int k = 0; k < need_c; ++k) used[n++] = out->copiers[k] = static_cast<hipStream_t>(s->copiers[k]);
  for (int a = 0; a < n; ++a)
    for (int b = a + 1; b < n; ++b)
      if (used[a] == used[b])
        return fail(TPSLICE_ERR_INVALID, "the call's streams must differ (the caller, %d worker and %d copy "
                    "stream(s); positions %d and %d are the same stream)", need_w, need_c, a, b);
  out->have_copiers = need_c > 0;
  // Graph capture is supported for joined plans with one worker stream. A pipelined call waits for
  // events of earlier calls, and capturing a plan with more worker streams has crashed the HIP
  // runtime while it ended the capture; both are refused before anything is queued.
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  const hipError_t qe = hipStreamIsCapturing(out->caller, &st);
  if (qe != hipSuccess) (void)hipGetLastError();  // a failed query must not read as the next launch's error
  out->capturing = qe == hipSuccess && st != hipStreamCaptureStatusNone;
  if (out->capturing && (p->S > 1 || (p->desc.flags & TPSLICE_F_PIPELINE)))
    return fail(TPSLICE_ERR_UNSUPPORTED, "the caller's stream is capturing a graph: only a plan with one worker "
                "stream and no pipelining can be captured (this one: %d worker streams%s)", p->S,
                (p->desc.flags & TPSLICE_F_PIPELINE) ? ", pipelined" : "");
  return TPSLICE_OK;
}

Schedule schedule(tpslice_plan_s* p, Runtime* rt, const CallStreams& cs) {
  Schedule S{p, rt, cs.caller, cs.serial, cs.workers, cs.have_copiers ? cs.copiers : nullptr};
  S.capturing = cs.capturing;
  return S;
}

GemmArgs args(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int64_t M,
              int64_t N, int64_t K) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = int32_t(M); g.N = int32_t(N); g.K = int32_t(K);
  return g;
}

const char* bf(const void* p, int64_t elems) { return static_cast<const char*>(p) + elems * 2; }
char* bfw(void* p, int64_t elems) { return static_cast<char*>(p) + elems * 2; }

tpslice_status_t check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return TPSLICE_OK;
  if (!ws) return fail(TPSLICE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign)
    return fail(TPSLICE_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kWsAlign);
  if (have < need) return fail(TPSLICE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return TPSLICE_OK;
}

#define TPS_REQ(ptr)                                                                  \
  do {                                                                                \
    if (!(ptr)) return fail(TPSLICE_ERR_INVALID, "%s is NULL", #ptr);                 \
    if (!aligned16(ptr)) return fail(TPSLICE_ERR_INVALID, "%s is not 16-byte aligned", #ptr); \
  } while (0)
#define TPS_OPT(ptr)                                                                  \
  do {                                                                                \
    if ((ptr) && !aligned16(ptr)) return fail(TPSLICE_ERR_INVALID, "%s is not 16-byte aligned", #ptr); \
  } while (0)
#define TPS_TRY(x)                       \
  do {                                           \
    tpslice_status_t st_ = (x);                  \
    if (st_ != TPSLICE_OK) return st_;           \
  } while (0)

}  // namespace
}  // namespace tps

using namespace tps;

extern "C" tpslice_status_t tpslice_plan_destroy(tpslice_plan_t p) {
  clear_error();
  if (!p) return TPSLICE_OK;
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  destroy_runtime(static_cast<Runtime*>(p->rt));
  p->rt = nullptr;
  p->magic = kDeadMagic;
  delete p;
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_mlp_fwd(tpslice_plan_t p, const void* X, const void* W1, const void* b1,
                                            const void* W2, void* Z, void* U_save, void* Z_handoff, void* ws,
                                            size_t ws_bytes, const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  TPS_REQ(W1); TPS_REQ(W2);
  if (p->M > 0) { TPS_REQ(X); TPS_REQ(Z); } else { TPS_OPT(X); TPS_OPT(Z); }
  TPS_OPT(b1); TPS_OPT(U_save); TPS_OPT(Z_handoff);
  const MlpFwdWs L = mlp_fwd_ws(p);
  TPS_TRY(check_ws(ws, ws_bytes, L.total));
  CallStreams cs;
  TPS_TRY(call_streams(p, streams, Z_handoff != nullptr, &cs));
  if (p->M == 0) return TPSLICE_OK;
  Runtime* rt = nullptr;
  TPS_TRY(ensure_runtime(p, &rt));
  Schedule S = schedule(p, rt, cs);
  char* H = static_cast<char*>(ws) + L.H;
  const int epi = p->desc.act == TPSLICE_ACT_GELU ? kEpiGelu : kEpiSwiglu;
  TPS_TRY(S.fork());
  for (int i = 0; i < p->r; ++i) {
    const int64_t r0 = int64_t(i) * p->Ms;
    const bool group = i % p->gup == 0;  // row slice i starts an up-projection group
    TPS_TRY(S.slice_begin(i, group ? p->gup : 1));
    S.slice_streams = 0;
    if (group) {
      const int64_t rows = std::min<int64_t>(p->gup, p->r - i) * p->Ms;
      GemmArgs g1 = args(bf(X, r0 * p->h), p->h, W1, p->h, bfw(H, r0 * p->Fp), p->Fp, rows, p->Fp, p->h);
      g1.bias = b1;
      g1.half = p->Fp;
      if (U_save) { g1.aux_out = bfw(U_save, r0 * p->N1); g1.ld_out = p->N1; }
      TPS_TRY(S.product_split(i, TPSLICE_STEP_MLP_UP, -1, g1, kFwd, epi, p->sp_up,
                              S.slice_part(static_cast<char*>(ws) + L.up_split, L.up_split_bytes, i)));
    }
    for (int j = 0; j < p->pc; ++j) {
      const int64_t c0 = int64_t(j) * p->pw;
      GemmArgs g2 = args(bf(H, r0 * p->Fp), p->Fp, bf(W2, c0 * p->Fp), p->Fp, bfw(Z, r0 * p->h + c0), p->h,
                         p->Ms, p->pw, p->Fp);
      TPS_TRY(S.product(i, TPSLICE_STEP_MLP_DOWN, j, g2, kFwd, kEpiBf16, 0, false, Z_handoff != nullptr));
      if (Z_handoff) TPS_TRY(S.handoff(i, j, Z, Z_handoff));
    }
    TPS_TRY(S.slice_handed_off(i, S.slice_streams));
  }
  return S.join();
}

extern "C" tpslice_status_t tpslice_attnproj_fwd(tpslice_plan_t p, const void* X, const void* Wqkv,
                                                 const void* bqkv, void* QKV, const void* C, const void* Wo,
                                                 void* Z, void* Z_handoff, void* ws, size_t ws_bytes,
                                                 const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (p->qh == 0) return fail(TPSLICE_ERR_UNSUPPORTED, "the plan has no attention heads (n_heads = 0)");
  // Wqkv NULL: no QKV projection (X, bqkv, QKV unused); Wo NULL: no output projection (C, Z,
  // Z_handoff unused), e.g. with the attention core between the two
  const bool do_qkv = Wqkv != nullptr, do_out = Wo != nullptr;
  if (!do_qkv && !do_out) return fail(TPSLICE_ERR_INVALID, "Wqkv and Wo are both NULL: nothing to compute");
  if (do_qkv) {
    TPS_REQ(Wqkv);
    if (p->M > 0) { TPS_REQ(X); TPS_REQ(QKV); } else { TPS_OPT(X); TPS_OPT(QKV); }
    TPS_OPT(bqkv);
  }
  if (do_out) {
    TPS_REQ(Wo);
    if (p->M > 0) { TPS_REQ(C); TPS_REQ(Z); } else { TPS_OPT(C); TPS_OPT(Z); }
    TPS_OPT(Z_handoff);
  } else {
    Z_handoff = nullptr;
  }
  const AttnFwdWs L = attn_fwd_ws(p);
  TPS_TRY(check_ws(ws, ws_bytes, L.total));
  CallStreams cs;
  TPS_TRY(call_streams(p, streams, Z_handoff != nullptr, &cs));
  if (p->M == 0) return TPSLICE_OK;
  Runtime* rt = nullptr;
  TPS_TRY(ensure_runtime(p, &rt));
  Schedule S = schedule(p, rt, cs);
  TPS_TRY(S.fork());
  // the output projection by row slices: its pieces are the hand-off
  for (int i = 0; do_out && i < p->r; ++i) {
    const int64_t r0 = int64_t(i) * p->Ms;
    TPS_TRY(S.slice_begin(i));
    S.slice_streams = 0;
    for (int j = 0; j < p->pc; ++j) {
      const int64_t c0 = int64_t(j) * p->pw;
      GemmArgs g = args(bf(C, r0 * p->ctx), p->ctx, bf(Wo, c0 * p->ctx), p->ctx, bfw(Z, r0 * p->h + c0), p->h,
                        p->Ms, p->pw, p->ctx);
      TPS_TRY(S.product(i, TPSLICE_STEP_OUT, j, g, kFwd, kEpiBf16, 0, false, Z_handoff != nullptr));
      if (Z_handoff) TPS_TRY(S.handoff(i, j, Z, Z_handoff));
    }
    TPS_TRY(S.slice_handed_off(i, S.slice_streams));
  }
  // QKV over all tokens at once, under the last pieces' copies: nothing hands it off and nothing in
  // this call reads it, so slicing it would only cut it into products too small to fill the GPU
  // (the 70B shard's 2048-row slices made 8 x 5 tiles of 256 x 256 each)
  if (do_qkv) {
    if (do_out) TPS_TRY(S.gather_slices());
    else TPS_TRY(S.wait_all_handoffs(0));
    GemmArgs q = args(X, p->h, Wqkv, p->h, QKV, p->qkv, p->M, p->qkv, p->h);
    q.bias = bqkv;
    TPS_TRY(S.product_split(-1, TPSLICE_STEP_QKV, -1, q, kFwd, kEpiBf16, p->sp_qkv,
                            reinterpret_cast<float*>(static_cast<char*>(ws) + L.qkv_split), 0, true));
  }
  return S.join();
}

extern "C" tpslice_status_t tpslice_mlp_bwd(tpslice_plan_t p, const void* X, const void* W1, const void* W2,
                                            const void* U, const void* dY, void* dX, void* dX_handoff,
                                            float* dW1, float* db1, float* dW2, int32_t accumulate, void* ws,
                                            size_t ws_bytes, const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  TPS_REQ(W1); TPS_REQ(W2); TPS_REQ(dW1); TPS_REQ(dW2);
  if (p->M > 0) { TPS_REQ(X); TPS_REQ(U); TPS_REQ(dY); TPS_REQ(dX); }
  else { TPS_OPT(X); TPS_OPT(U); TPS_OPT(dY); TPS_OPT(dX); }
  TPS_OPT(db1); TPS_OPT(dX_handoff);
  if (accumulate != 0 && accumulate != 1) return fail(TPSLICE_ERR_INVALID, "accumulate must be 0 or 1");
  const MlpBwdWs L = mlp_bwd_ws(p);
  TPS_TRY(check_ws(ws, ws_bytes, L.total));
  CallStreams cs;
  TPS_TRY(call_streams(p, streams, dX_handoff != nullptr, &cs));
  Runtime* rt = nullptr;
  TPS_TRY(ensure_runtime(p, &rt));
  Schedule S = schedule(p, rt, cs);
  char* dU = static_cast<char*>(ws) + L.dU;
  char* H = static_cast<char*>(ws) + L.H;
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + L.partials);
  const bool glu = p->desc.act == TPSLICE_ACT_SWIGLU;
  TPS_TRY(S.fork());
  for (int i = 0; i < p->r && p->M > 0; ++i) {
    const int64_t r0 = int64_t(i) * p->Ms;
    const bool group = i % p->gdh == 0;  // row slice i starts a dH group
    TPS_TRY(S.slice_begin(i, group ? p->gdh : 1));
    S.slice_streams = 0;
    if (group) {
      // dH = dY W2 with the activation's derivative fused, over the group's rows: writes dU and
      // (recomputed) H
      const int64_t rows = std::min<int64_t>(p->gdh, p->r - i) * p->Ms;
      GemmArgs g = args(bf(dY, r0 * p->h), p->h, W2, p->Fp, bfw(dU, r0 * p->N1), p->N1, rows, p->Fp, p->h);
      g.aux_in = bf(U, r0 * p->N1); g.ld_in = p->N1;
      g.aux_out = bfw(H, r0 * p->Fp); g.ld_out = p->Fp;
      g.half = p->Fp;
      TPS_TRY(S.product_split(i, TPSLICE_STEP_MLP_DH, -1, g, kDgrad, glu ? kEpiDswiglu : kEpiDgelu, p->sp_dh,
                              S.slice_part(static_cast<char*>(ws) + L.dh_split, L.dh_split_bytes, i)));
    }
    for (int j = 0; j < p->pc; ++j) {
      const int64_t c0 = int64_t(j) * p->pw;
      GemmArgs gx = args(bf(dU, r0 * p->N1), p->N1, bf(W1, c0), p->h, bfw(dX, r0 * p->h + c0), p->h, p->Ms, p->pw,
                         p->N1);
      TPS_TRY(S.product(i, TPSLICE_STEP_MLP_DX, j, gx, kDgrad, kEpiBf16, 0, false, dX_handoff != nullptr));
      if (dX_handoff) TPS_TRY(S.handoff(i, j, dX, dX_handoff));
    }
    TPS_TRY(S.slice_handed_off(i, S.slice_streams));
  }
  // weight gradients over all tokens at once (one k run, no split of the token sum), under the
  // last pieces' copies, one after another on worker 0 (side by side on two workers each took half
  // the CUs for the same total time)
  TPS_TRY(S.gather_slices());
  GemmArgs g1 = args(dU, p->N1, X, p->h, dW1, p->h, p->N1, p->h, p->M);
  g1.accumulate = accumulate;
  TPS_TRY(S.product_split(-1, TPSLICE_STEP_MLP_DW1, -1, g1, kWgrad, kEpiF32, p->sp_dw1,
                          reinterpret_cast<float*>(static_cast<char*>(ws) + L.dw1_split), 0, false, p->tl_dw1));
  GemmArgs g2 = args(dY, p->h, H, p->Fp, dW2, p->Fp, p->h, p->Fp, p->M);
  g2.accumulate = accumulate;
  TPS_TRY(S.product_split(-1, TPSLICE_STEP_MLP_DW2, -1, g2, kWgrad, kEpiF32, p->sp_dw2,
                          reinterpret_cast<float*>(static_cast<char*>(ws) + L.dw2_split), 0, false, p->tl_dw2));
  if (db1) TPS_TRY(S.colsum(dU, p->N1, p->M, p->N1, partials, db1, accumulate, 0));
  return S.join();
}

// Checks shared by the attention core's entry points (before anything is queued).
static tpslice_status_t check_attn_core(const tpslice_plan_s* p, int64_t seq_len) {
  if (!p->qh) return fail(TPSLICE_ERR_UNSUPPORTED, "the plan has no attention heads");
  if (p->desc.head_dim != kAttnHeadDim)
    return fail(TPSLICE_ERR_UNSUPPORTED, "head_dim %d: the attention core takes %d", p->desc.head_dim, kAttnHeadDim);
  if (seq_len <= 0 || seq_len % kAttnBlock != 0 || seq_len > (int64_t(1) << 30) || p->M % seq_len != 0)
    return fail(TPSLICE_ERR_SHAPE, "seq_len %lld must be a positive multiple of %d dividing the %lld tokens",
                (long long)seq_len, kAttnBlock, (long long)p->M);
  if (p->qh % p->kvh != 0) return fail(TPSLICE_ERR_SHAPE, "%d query heads over %d kv heads", p->qh, p->kvh);
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_attn_core_fwd(tpslice_plan_t p, const void* QKV, void* C, float* lse,
                                                  int64_t seq_len, const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (p->M > 0) { TPS_REQ(QKV); TPS_REQ(C); } else { TPS_OPT(QKV); TPS_OPT(C); }
  TPS_OPT(lse);
  TPS_TRY(check_attn_core(p, seq_len));
  if (p->M == 0) return TPSLICE_OK;
  AttnArgs a{QKV, C, lse, p->qkv, p->ctx, p->M, int32_t(seq_len), p->qh, p->kvh,
             float(1.4426950408889634 / std::sqrt(double(kAttnHeadDim)))};
  hipError_t e = launch_attn_fwd(a, streams ? static_cast<hipStream_t>(streams->caller) : nullptr);
  if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_attn_core_bwd(tpslice_plan_t p, const void* QKV, const void* C,
                                                  const float* lse, const void* dC, void* dQKV, int64_t seq_len,
                                                  void* ws, size_t ws_bytes, const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (p->M > 0) { TPS_REQ(QKV); TPS_REQ(C); TPS_REQ(lse); TPS_REQ(dC); TPS_REQ(dQKV); }
  else { TPS_OPT(QKV); TPS_OPT(C); TPS_OPT(lse); TPS_OPT(dC); TPS_OPT(dQKV); }
  TPS_TRY(check_attn_core(p, seq_len));
  TPS_TRY(check_ws(ws, ws_bytes, attn_bwd_workspace_bytes(p->M, p->qh, p->kvh)));
  if (p->M == 0) return TPSLICE_OK;
  const double sc = 1.0 / std::sqrt(double(kAttnHeadDim));
  AttnBwdArgs a{QKV, C, dC, lse, dQKV, nullptr, nullptr, p->qkv, p->ctx, p->M, int32_t(seq_len), p->qh, p->kvh,
                float(sc), float(1.4426950408889634 * sc)};
  hipError_t e = launch_attn_bwd(a, ws, streams ? static_cast<hipStream_t>(streams->caller) : nullptr);
  if (e != hipSuccess) return fail(TPSLICE_ERR_HIP, "attention backward launch: %s", hipGetErrorString(e));
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_attnproj_bwd(tpslice_plan_t p, const void* X, const void* Wqkv,
                                                 const void* dQKV, const void* C, const void* Wo, const void* dY,
                                                 void* dX, void* dX_handoff, void* dC, float* dWqkv,
                                                 float* dbqkv, float* dWo, int32_t accumulate, void* ws,
                                                 size_t ws_bytes, const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (p->qh == 0) return fail(TPSLICE_ERR_UNSUPPORTED, "the plan has no attention heads (n_heads = 0)");
  // Wo NULL: no output-projection gradients (C, dY, dC, dWo unused); Wqkv NULL: no QKV-projection
  // gradients (X, dQKV, dX, dX_handoff, dWqkv, dbqkv unused). With the attention core between them,
  // the first half gives dC for the core's backward, whose dQKV the second half takes.
  const bool do_out = Wo != nullptr, do_qkv = Wqkv != nullptr;
  if (!do_qkv && !do_out) return fail(TPSLICE_ERR_INVALID, "Wqkv and Wo are both NULL: nothing to compute");
  if (do_out) {
    TPS_REQ(Wo); TPS_REQ(dWo);
    if (p->M > 0) { TPS_REQ(C); TPS_REQ(dY); TPS_REQ(dC); } else { TPS_OPT(C); TPS_OPT(dY); TPS_OPT(dC); }
  }
  if (do_qkv) {
    TPS_REQ(Wqkv); TPS_REQ(dWqkv);
    if (p->M > 0) { TPS_REQ(X); TPS_REQ(dQKV); TPS_REQ(dX); } else { TPS_OPT(X); TPS_OPT(dQKV); TPS_OPT(dX); }
    TPS_OPT(dbqkv); TPS_OPT(dX_handoff);
  } else {
    dX_handoff = nullptr;
    dbqkv = nullptr;
  }
  if (accumulate != 0 && accumulate != 1) return fail(TPSLICE_ERR_INVALID, "accumulate must be 0 or 1");
  const AttnBwdWs L = attn_bwd_ws(p);
  TPS_TRY(check_ws(ws, ws_bytes, L.total));
  CallStreams cs;
  TPS_TRY(call_streams(p, streams, dX_handoff != nullptr, &cs));
  Runtime* rt = nullptr;
  TPS_TRY(ensure_runtime(p, &rt));
  Schedule S = schedule(p, rt, cs);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + L.partials);
  TPS_TRY(S.fork());
  for (int i = 0; i < p->r && p->M > 0 && do_qkv; ++i) {
    const int64_t r0 = int64_t(i) * p->Ms;
    TPS_TRY(S.slice_begin(i));
    S.slice_streams = 0;
    for (int j = 0; j < p->pc; ++j) {
      const int64_t c0 = int64_t(j) * p->pw;
      GemmArgs gx = args(bf(dQKV, r0 * p->qkv), p->qkv, bf(Wqkv, c0), p->h, bfw(dX, r0 * p->h + c0), p->h, p->Ms,
                         p->pw, p->qkv);
      TPS_TRY(S.product(i, TPSLICE_STEP_ATTN_DX, j, gx, kDgrad, kEpiBf16, 0, false, dX_handoff != nullptr));
      if (dX_handoff) TPS_TRY(S.handoff(i, j, dX, dX_handoff));
    }
    TPS_TRY(S.slice_handed_off(i, S.slice_streams));
  }
  // dC is handed to the attention core, not off the GPU: it runs over all tokens (narrow output,
  // so the whole batch fills the CUs better than a slice), then the weight gradients, one after
  // another on worker 0 (measured on the Llama-3 70B shard: side by side on two workers, each at
  // half the CUs, they took 0.81 ms against 0.74 ms in sequence)
  TPS_TRY(S.gather_slices());
  if (!do_qkv) TPS_TRY(S.wait_all_handoffs(0));
  if (do_out) {
    if (p->M > 0) {
      GemmArgs gc = args(dY, p->h, Wo, p->ctx, dC, p->ctx, p->M, p->ctx, p->h);
      TPS_TRY(S.product_split(-1, TPSLICE_STEP_ATTN_DC, -1, gc, kDgrad, kEpiBf16, p->sp_dc,
                              reinterpret_cast<float*>(static_cast<char*>(ws) + L.dc_split), 0));
    }
    GemmArgs go = args(dY, p->h, C, p->ctx, dWo, p->ctx, p->h, p->ctx, p->M);
    go.accumulate = accumulate;
    TPS_TRY(S.product_split(-1, TPSLICE_STEP_ATTN_DWO, -1, go, kWgrad, kEpiF32, p->sp_dwo,
                            reinterpret_cast<float*>(static_cast<char*>(ws) + L.dwo_split), 0, false, p->tl_dwo));
  }
  if (do_qkv) {
    GemmArgs gq = args(dQKV, p->qkv, X, p->h, dWqkv, p->h, p->qkv, p->h, p->M);
    gq.accumulate = accumulate;
    TPS_TRY(S.product_split(-1, TPSLICE_STEP_ATTN_DWQKV, -1, gq, kWgrad, kEpiF32, p->sp_dwqkv,
                            reinterpret_cast<float*>(static_cast<char*>(ws) + L.dwqkv_split), 0, false,
                            p->tl_dwqkv));
    if (dbqkv) TPS_TRY(S.colsum(dQKV, p->qkv, p->M, p->qkv, partials, dbqkv, accumulate, 0));
  }
  return S.join();
}

extern "C" tpslice_status_t tpslice_trace_enable(tpslice_plan_t p, int32_t enable) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (enable < 0 || enable > 3) return fail(TPSLICE_ERR_INVALID, "trace mask %d outside [0, 3]", enable);
  p->trace = enable;
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_trace_read(tpslice_plan_t p, tpslice_trace_rec_t* recs, int32_t cap,
                                               int32_t* count) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (!count || (cap > 0 && !recs)) return fail(TPSLICE_ERR_INVALID, "recs/count is NULL");
  if (!p->trace) return fail(TPSLICE_ERR_INVALID, "tracing is not enabled on this plan");
  Runtime* rt = static_cast<Runtime*>(p->rt);
  *count = 0;
  if (!rt || !rt->window_open) return TPSLICE_OK;
  *count = int32_t(rt->slots.size());
  if (cap < *count) return TPSLICE_OK;
  for (size_t k = 0; k < rt->slots.size(); ++k) {
    TraceSlot& t = rt->slots[k];
    TPS_HIP(hipEventSynchronize(rt->tpool[t.ev1]));
    float a = 0.f, b = 0.f;
    TPS_HIP(hipEventElapsedTime(&a, rt->t0, rt->tpool[t.ev0]));
    TPS_HIP(hipEventElapsedTime(&b, rt->t0, rt->tpool[t.ev1]));
    t.rec.start_ms = a;
    t.rec.end_ms = b;
    recs[k] = t.rec;
  }
  rt->slots.clear();
  rt->tused = 0;
  rt->window_open = false;
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_handoff_wait(tpslice_plan_t p, void* stream) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  Runtime* rt = static_cast<Runtime*>(p->rt);
  if (!rt) return TPSLICE_OK;
  // a pipelined call leaves the end of each row slice's copies in `copied`; other calls join
  // their copies before they return
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (size_t x = 0; x < rt->copied.size(); ++x)
    if (rt->copied_pending[x]) TPS_HIP(hipStreamWaitEvent(s, rt->copied[x], 0));
  return TPSLICE_OK;
}

extern "C" tpslice_status_t tpslice_handoff_copy(tpslice_plan_t p, const void* src, void* dst,
                                                const tpslice_streams_t* streams) {
  clear_error();
  if (!plan_ok(p)) return fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  if (p->M > 0) { TPS_REQ(src); TPS_REQ(dst); }
  CallStreams cs;
  TPS_TRY(call_streams(p, streams, true, &cs));
  if (p->M == 0) return TPSLICE_OK;
  Runtime* rt = nullptr;
  TPS_TRY(ensure_runtime(p, &rt));
  Schedule S = schedule(p, rt, cs);
  TPS_TRY(S.fork());
  for (int i = 0; i < p->r; ++i) {
    TPS_TRY(S.slice_begin(i));
    S.slice_streams = 0;
    for (int j = 0; j < p->pc; ++j) TPS_TRY(S.handoff(i, j, src, dst));
    TPS_TRY(S.slice_handed_off(i, S.slice_streams));
  }
  return S.join();
}
