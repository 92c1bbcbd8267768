// extern "C" entry points of libblockrank (declared in include/blockrank.h).
//
// Each compute call: validate everything on the host, build the work plan, copy the plan into
// the caller's workspace through a pinned staging buffer (a small copy kernel on the caller's
// stream), then enqueue the kernels on that stream.  Nothing blocks the host except the first
// use of a staging buffer size (pinned allocation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <list>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "blockrank.h"
#include "launch.h"
#include "plan.h"

namespace br {
// Plan copy on the compute queue: the kernel reads the pinned staging buffer over PCIe.  A
// host-to-device hipMemcpyAsync of the same bytes runs on a DMA engine and costs a
// cross-engine synchronisation (tens of microseconds) before the kernel that reads the plan.
__global__ __launch_bounds__(256) void plan_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256) dst[i] = src[i];
}

}  // namespace br

namespace {

thread_local std::string g_last_error;

br_status record(const br::Error& e) {
  g_last_error = e.msg;
  return e.status;
}
br_status record(br_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
br_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return BR_ERR_HIP;
}

// Pinned host buffers for plan uploads.  A buffer is reused once the copy that read it is known
// to have completed.  Recording an event between two kernels costs the stream a few
// microseconds, so events are batched: buffers released on a stream stay pending until
// kEventBatch of them have accumulated (or the pool has grown large), then one event recorded
// on that stream covers them all (the copies that read them precede it in stream order).
class StagingPool {
 public:
  struct Lease {
    int index = -1;
    void* ptr = nullptr;
  };

  hipError_t acquire(size_t bytes, Lease* lease) {
    std::lock_guard<std::mutex> lock(mu_);
    hipError_t e = retire_completed();
    if (e != hipSuccess) return e;
    for (size_t i = 0; i < bufs_.size(); ++i) {
      Buf& b = bufs_[i];
      if (b.state != kFree || b.cap < bytes) continue;
      b.state = kBusy;
      *lease = Lease{int(i), b.host};
      return hipSuccess;
    }
    Buf nb;
    nb.cap = bytes < (size_t(64) << 10) ? (size_t(64) << 10) : bytes;
    e = hipHostMalloc(&nb.host, nb.cap, hipHostMallocDefault);
    if (e != hipSuccess) return e;
    nb.state = kBusy;
    bufs_.push_back(nb);
    *lease = Lease{int(bufs_.size() - 1), nb.host};
    return hipSuccess;
  }

  // The lease's contents are read by work already enqueued on `stream` (if `enqueued`).
  hipError_t release(const Lease& lease, hipStream_t stream, bool enqueued) {
    std::lock_guard<std::mutex> lock(mu_);
    Buf& b = bufs_[size_t(lease.index)];
    if (!enqueued) {
      b.state = kFree;
      return hipSuccess;
    }
    b.state = kPending;
    b.stream = stream;
    int pending = 0;
    for (const Buf& x : bufs_) pending += x.state == kPending && x.stream == stream;
    if (pending < kEventBatch && bufs_.size() < kMaxBufs) return hipSuccess;
    // One event after the copies that read every pending buffer of this stream.
    hipEvent_t ev = nullptr;
    hipError_t e = take_event(&ev);
    if (e != hipSuccess) return e;
    e = hipEventRecord(ev, stream);
    if (e != hipSuccess) {
      events_free_.push_back(ev);
      return e;
    }
    for (size_t i = 0; i < bufs_.size(); ++i)
      if (bufs_[i].state == kPending && bufs_[i].stream == stream) {
        bufs_[i].state = kCovered;
        bufs_[i].event_slot = int(inflight_.size());
      }
    inflight_.push_back(ev);
    return hipSuccess;
  }

 private:
  static constexpr int kEventBatch = 4;
  static constexpr size_t kMaxBufs = 32;
  enum State { kFree, kBusy, kPending, kCovered };
  struct Buf {
    void* host = nullptr;
    size_t cap = 0;
    State state = kFree;
    hipStream_t stream = nullptr;
    int event_slot = -1;  // index into inflight_ while kCovered
  };

  hipError_t take_event(hipEvent_t* ev) {
    if (!events_free_.empty()) {
      *ev = events_free_.back();
      events_free_.pop_back();
      return hipSuccess;
    }
    // Only completion matters (the host reads nothing back): a device-scope release avoids a
    // cache writeback when the event is recorded.
    return hipEventCreateWithFlags(ev, hipEventDisableTiming | hipEventReleaseToDevice);
  }

  // Free the buffers whose covering event has completed; recycle those events.
  hipError_t retire_completed() {
    std::vector<hipEvent_t> keep;
    std::vector<int> remap(inflight_.size(), -1);
    for (size_t k = 0; k < inflight_.size(); ++k) {
      const hipError_t q = hipEventQuery(inflight_[k]);
      if (q == hipSuccess) {
        events_free_.push_back(inflight_[k]);
      } else if (q == hipErrorNotReady) {
        remap[k] = int(keep.size());
        keep.push_back(inflight_[k]);
      } else {
        return q;
      }
    }
    for (Buf& b : bufs_) {
      if (b.state != kCovered) continue;
      const int slot = remap[size_t(b.event_slot)];
      if (slot < 0) {
        b.state = kFree;
        b.event_slot = -1;
      } else {
        b.event_slot = slot;
      }
    }
    inflight_.swap(keep);
    return hipSuccess;
  }

  std::mutex mu_;
  std::vector<Buf> bufs_;                 // kept for the life of the process
  std::vector<hipEvent_t> inflight_;      // recorded, not yet known complete
  std::vector<hipEvent_t> events_free_;   // completed, reusable
};

StagingPool& staging() {
  static StagingPool* pool = new StagingPool();  // intentionally never destroyed
  return *pool;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Copy `bytes` from `src` (host) into device memory `dst` on `stream` via pinned staging.
br_status upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return BR_OK;
  StagingPool::Lease lease;
  hipError_t e = staging().acquire(bytes, &lease);
  if (e != hipSuccess) return hip_fail(e, "pinned staging allocation");
  std::memcpy(lease.ptr, src, bytes);
  void* dsrc = nullptr;
  if (bytes % 16 == 0 && aligned(dst, 16) && hipHostGetDevicePointer(&dsrc, lease.ptr, 0) == hipSuccess) {
    const size_t n16 = bytes / 16;
    const unsigned blocks = unsigned(std::min<size_t>(64, (n16 + 255) / 256));
    br::plan_copy_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint4*>(dsrc), static_cast<uint4*>(dst), n16);
    e = hipGetLastError();
  } else {
    e = hipMemcpyAsync(dst, lease.ptr, bytes, hipMemcpyHostToDevice, stream);
  }
  hipError_t r = staging().release(lease, stream, e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "plan upload");
  if (r != hipSuccess) return hip_fail(r, "plan upload (hipEventRecord)");
  return BR_OK;
}

// Persistent attention workgroup slots of the current device (CUs x workgroups per CU), cached
// per device.  Host-only queries (workspace sizing, plan introspection) use kDefaultCus.
constexpr int kDefaultCus = 256;
hipError_t attn_workgroups(int* out) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (size_t(dev) >= cache.size()) cache.resize(size_t(dev) + 1, 0);
  if (cache[size_t(dev)] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[size_t(dev)] = (cus > 0 ? cus : kDefaultCus) * br::kAttnWgPerCu;
  }
  *out = cache[size_t(dev)];
  return hipSuccess;
}


// Token count from which the ranking step runs its readout beside the attention (measured on
// MI355X: 3% faster at 100,096 tokens, 1.4% at 16 x 13,500 and 3% at 30,407; 14% slower at 12,864).
constexpr int64_t kSideStreamMinTokens = 24576;

// A second stream per device for the ranking step's readout, which depends only on the inputs
// and runs beside the attention: forked from and joined back to the caller's stream with two
// events.  Default priority; created on first use and kept until the process ends.  `lock` is
// held while a call enqueues its fork, readout and join, so calls from several host threads
// never interleave their use of the shared events.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex lock;
};
hipError_t side_stream(SideStream** out) {
  static std::mutex mu;
  static std::vector<SideStream*> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> guard(mu);
  if (size_t(dev) >= per_device.size()) per_device.resize(size_t(dev) + 1, nullptr);
  if (!per_device[size_t(dev)]) {
    SideStream* s = new SideStream;
    e = hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (s->join) (void)hipEventDestroy(s->join);
      if (s->fork) (void)hipEventDestroy(s->fork);
      if (s->stream) (void)hipStreamDestroy(s->stream);
      delete s;
      return e;
    }
    per_device[size_t(dev)] = s;
  }
  *out = per_device[size_t(dev)];
  return hipSuccess;
}

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / std::sqrt(float(d)); }

template <class F>
br_status guarded(F&& f) {
  try {
    return f();
  } catch (const std::exception& ex) {
    return record(BR_ERR_INVALID_ARG, std::string("internal error: ") + ex.what());
  } catch (...) {
    return record(BR_ERR_INVALID_ARG, "internal error");
  }
}

// Buffer checks shared by the attention entry points (host only).
br_status check_attn_buffers(const void* Q, const void* K, const void* V, const void* out, const float* lse,
                             float softmax_scale) {
  if (!Q || !K || !V || !out) return record(BR_ERR_INVALID_ARG, "Q, K, V and out must be non-NULL device pointers");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16))
    return record(BR_ERR_INVALID_ARG, "Q, K, V and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return record(BR_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
    return record(BR_ERR_INVALID_ARG, "softmax_scale must be finite");
  return BR_OK;
}

// Upload a validated attention plan into the workspace and launch it.  Q, out and lse rows are
// addressed relative to token q_row_base.
// The fused rotation's cos/sin table covers each distinct position once: the rotation runs
// (instruction, each document, query) of all prompts merged into intervals of consecutive
// positions; table row = interval offset + position - interval start.
struct RopeTable {
  std::vector<int32_t> iv_pos0, iv_off, run_row0;
  int64_t rows = 0;
  size_t off_pidx = 0, off_ivp = 0, off_ivo = 0, off_freq = 0, off_table = 0, bytes = 0;  // after the plan
};

void build_rope_table(const br::RopePlan& rp, int head_dim, size_t n_items, RopeTable* t) {
  const size_t nr = rp.pos0.size();
  std::vector<std::pair<int64_t, int64_t>> spans(nr);
  for (size_t r = 0; r < nr; ++r) spans[r] = {rp.pos0[r], int64_t(rp.pos0[r]) + (rp.start[r + 1] - rp.start[r])};
  std::sort(spans.begin(), spans.end());
  t->iv_pos0.clear();
  t->iv_off.clear();
  int64_t cur0 = 0, cur1 = -1;
  for (const auto& sp : spans) {
    if (cur1 >= 0 && sp.first <= cur1) {
      cur1 = std::max(cur1, sp.second);
      continue;
    }
    if (cur1 >= 0) {
      t->iv_pos0.push_back(int32_t(cur0));
      t->iv_off.push_back(int32_t(t->rows));
      t->rows += cur1 - cur0;
    }
    cur0 = sp.first;
    cur1 = sp.second;
  }
  if (cur1 >= 0) {
    t->iv_pos0.push_back(int32_t(cur0));
    t->iv_off.push_back(int32_t(t->rows));
    t->rows += cur1 - cur0;
  }
  t->run_row0.resize(nr);
  for (size_t r = 0; r < nr; ++r) {
    const size_t i = size_t(std::upper_bound(t->iv_pos0.begin(), t->iv_pos0.end(), rp.pos0[r]) - t->iv_pos0.begin()) - 1;
    t->run_row0[r] = t->iv_off[i] + (rp.pos0[r] - t->iv_pos0[i]);
  }
  const size_t niv = t->iv_pos0.size();
  t->off_pidx = 0;
  t->off_ivp = br::align_up(n_items * 4, 256);
  t->off_ivo = t->off_ivp + br::align_up(niv * 4, 16);
  t->off_freq = t->off_ivo + br::align_up(niv * 4, 16);
  t->off_table = br::align_up(t->off_freq + size_t(head_dim / 2) * 8, 256);
  t->bytes = br::align_up(t->off_table + size_t(t->rows) * size_t(head_dim) * 4, 256);
}

br_status run_attn(const br_dims& dims, br::AttnPlan& plan, const void* Q, const void* K, const void* V, void* out,
                   float* lse, float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream,
                   int q_row_base, hipEvent_t kernel_start, hipEvent_t kernel_stop, bool pageable_upload = false,
                   float sink_log2 = -__builtin_inff(), const br::RopePlan* rope = nullptr, int rope_layout = 0) {
  RopeTable rt;
  if (rope) build_rope_table(*rope, dims.head_dim, plan.items.size(), &rt);
  const size_t need = plan.total_bytes + rt.bytes;
  if (!workspace || workspace_bytes < need)
    return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than the workspace size query's " +
                                        std::to_string(need) + " bytes");
  if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  // All arguments are valid: only now touch the runtime (device query for the schedule).
  int workgroups = 0;
  hipError_t he0 = attn_workgroups(&workgroups);
  if (he0 != hipSuccess) return hip_fail(he0, "device query");
  br::schedule_attn_plan(dims.num_kv_heads, workgroups, &plan);

  // Host image of the plan region of the workspace: [items | ranges | merges].
  std::vector<unsigned char> host(plan.off_part_o, 0);
  std::memcpy(host.data() + plan.off_items, plan.sched.data(), plan.sched.size() * sizeof(br::AttnItem));
  std::memcpy(host.data() + plan.off_ranges, plan.ranges.data(), plan.ranges.size() * sizeof(int32_t));
  if (!plan.merges.empty())
    std::memcpy(host.data() + plan.off_merges, plan.merges.data(), plan.merges.size() * sizeof(br::MergeItem));
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (pageable_upload) {
    // Straight from pageable host memory: the runtime has copied the source out before the call
    // returns, and nothing is allocated here.
    hipError_t ce = hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, stream);
    if (ce != hipSuccess) return hip_fail(ce, "plan upload");
  } else {
    br_status st = upload(ws, host.data(), host.size(), stream);
    if (st != BR_OK) return st;
  }

  br::AttnLaunch a;
  if (rope) {
    // Per scheduled item, the table row of its first token (an item lies in one segment, i.e. one
    // rotation run, whose positions are consecutive); then the intervals, frequencies and table.
    unsigned char* wr = ws + plan.total_bytes;
    std::vector<unsigned char> hx(rt.off_table, 0);
    int32_t* pidx = reinterpret_cast<int32_t*>(hx.data() + rt.off_pidx);
    for (size_t i = 0; i < plan.sched.size(); ++i) {
      const int32_t row0 = plan.sched[i].row0;
      const size_t r = size_t(std::upper_bound(rope->start.begin(), rope->start.end() - 1, row0) - rope->start.begin()) - 1;
      pidx[i] = rt.run_row0[r] + (row0 - rope->start[r]);
    }
    std::memcpy(hx.data() + rt.off_ivp, rt.iv_pos0.data(), rt.iv_pos0.size() * 4);
    std::memcpy(hx.data() + rt.off_ivo, rt.iv_off.data(), rt.iv_off.size() * 4);
    std::memcpy(hx.data() + rt.off_freq, rope->inv_freq.data(), rope->inv_freq.size() * 8);
    if (pageable_upload) {
      hipError_t ce = hipMemcpyAsync(wr, hx.data(), hx.size(), hipMemcpyHostToDevice, stream);
      if (ce != hipSuccess) return hip_fail(ce, "rotation table upload");
    } else {
      br_status st = upload(wr, hx.data(), hx.size(), stream);
      if (st != BR_OK) return st;
    }
    hipError_t te = br::launch_rope_table(reinterpret_cast<const int32_t*>(wr + rt.off_ivp),
                                          reinterpret_cast<const int32_t*>(wr + rt.off_ivo), int(rt.iv_pos0.size()),
                                          rt.rows, dims.head_dim, reinterpret_cast<const double*>(wr + rt.off_freq),
                                          reinterpret_cast<float*>(wr + rt.off_table), stream);
    if (te != hipSuccess) return hip_fail(te, "rotation table kernel launch");
    a.rope = rope_layout;
    a.rope_cs = reinterpret_cast<const float*>(wr + rt.off_table);
    a.item_pidx = reinterpret_cast<const int32_t*>(wr + rt.off_pidx);
  }
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.items = reinterpret_cast<const br::AttnItem*>(ws + plan.off_items);
  a.ranges = reinterpret_cast<const int32_t*>(ws + plan.off_ranges);
  a.merges = reinterpret_cast<const br::MergeItem*>(ws + plan.off_merges);
  a.part_o = reinterpret_cast<float*>(ws + plan.off_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + plan.off_part_ml);
  a.n_items = int64_t(plan.items.size());
  a.n_merges = int64_t(plan.merges.size());
  a.wg_per_head = plan.wg_per_head;
  a.num_q_heads = dims.num_q_heads;
  a.num_kv_heads = dims.num_kv_heads;
  a.head_dim = dims.head_dim;
  a.scale_log2 = resolve_scale(softmax_scale, dims.head_dim) * 1.4426950408889634f;
  a.q_row_base = q_row_base;
  a.sink_log2 = sink_log2;
  a.ev_start = kernel_start;
  a.ev_stop = kernel_stop;
  hipError_t he = br::launch_attn(a, stream);
  if (he != hipSuccess) return hip_fail(he, "attention kernel launch");
  return BR_OK;
}

// Upload a validated rotary-embedding plan into the workspace and launch the rotation.
br_status run_rope(const br_dims& dims, const int32_t* seg_ptr, const br::RopePlan& plan, const void* Q, void* Q_out,
                   int q_heads, const void* K, void* K_out, int k_heads, int32_t interleaved, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  if (interleaved != 0 && interleaved != 1) return record(BR_ERR_INVALID_ARG, "interleaved must be 0 or 1");
  if (!Q != !Q_out || !K != !K_out)
    return record(BR_ERR_INVALID_ARG, "an input and its output must both be given or both be NULL");
  if (!Q && !K) return record(BR_ERR_INVALID_ARG, "nothing to rotate: Q and K are both NULL");
  if ((Q && (!aligned(Q, 16) || !aligned(Q_out, 16))) || (K && (!aligned(K, 16) || !aligned(K_out, 16))))
    return record(BR_ERR_INVALID_ARG, "Q, K and their outputs must be 16-byte aligned");
  // the documented size (one run per segment), which bounds what this plan uses
  const size_t required = br::rope_workspace_bytes(int64_t(seg_ptr[dims.num_prompts]) - dims.num_prompts, dims.head_dim);
  if (!workspace || workspace_bytes < required)
    return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_rope_workspace_bytes() = " +
                                        std::to_string(required));
  if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  std::vector<unsigned char> host(plan.total_bytes, 0);  // a multiple of 16 bytes
  std::memcpy(host.data() + plan.off_start, plan.start.data(), plan.start.size() * sizeof(int32_t));
  std::memcpy(host.data() + plan.off_pos0, plan.pos0.data(), plan.pos0.size() * sizeof(int32_t));
  std::memcpy(host.data() + plan.off_freq, plan.inv_freq.data(), plan.inv_freq.size() * sizeof(double));
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  br_status st = upload(ws, host.data(), host.size(), stream);
  if (st != BR_OK) return st;
  br::RopeLaunch l;
  l.q = static_cast<const uint16_t*>(Q);
  l.q_out = static_cast<uint16_t*>(Q_out);
  l.k = static_cast<const uint16_t*>(K);
  l.k_out = static_cast<uint16_t*>(K_out);
  l.run_start = reinterpret_cast<const int32_t*>(ws + plan.off_start);
  l.run_pos0 = reinterpret_cast<const int32_t*>(ws + plan.off_pos0);
  l.inv_freq = reinterpret_cast<const double*>(ws + plan.off_freq);
  l.rows = plan.rows;
  l.n_runs = int(plan.pos0.size());
  l.q_heads = Q ? q_heads : 0;
  l.k_heads = K ? k_heads : 0;
  l.head_dim = dims.head_dim;
  l.adjacent = interleaved == 1;
  hipError_t he = br::launch_rope(l, stream);
  if (he != hipSuccess) return hip_fail(he, "rotary embedding kernel launch");
  return BR_OK;
}


// Workspace of the allocation-free attention entry point: a file-scope device array (one copy
// per GPU, held until the process ends).  Host code never uses the array's name as an address:
// the device address comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(BR_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (size_t(dev) >= per_device.size()) per_device.resize(size_t(dev) + 1, nullptr);
  if (!per_device[size_t(dev)]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[size_t(dev)] = p;
  }
  *out = per_device[size_t(dev)];
  return hipSuccess;
}

}  // namespace

extern "C" {

br_status br_attn_fwd_noalloc(const br_dims* dims, const void* Q, const void* K, const void* V,
                              const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                              float softmax_scale, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    if (plan.total_bytes > kNoAllocScratchBytes)
      return record(BR_ERR_UNSUPPORTED, "this segment table needs " + std::to_string(plan.total_bytes) +
                                            " bytes of workspace; br_attn_fwd_noalloc has " +
                                            std::to_string(kNoAllocScratchBytes) + " (use br_attn_fwd)");
    void* ws = nullptr;
    hipError_t he = scratch_address(&ws);
    if (he != hipSuccess) return hip_fail(he, "hipGetSymbolAddress(scratch)");
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, ws, kNoAllocScratchBytes, stream, 0, nullptr,
                    nullptr, /*pageable_upload=*/true);
  });
}

}  // extern "C"

extern "C" {

const char* br_status_string(br_status s) {
  switch (s) {
    case BR_OK: return "BR_OK";
    case BR_ERR_INVALID_ARG: return "BR_ERR_INVALID_ARG";
    case BR_ERR_UNSUPPORTED: return "BR_ERR_UNSUPPORTED";
    case BR_ERR_WORKSPACE: return "BR_ERR_WORKSPACE";
    case BR_ERR_HIP: return "BR_ERR_HIP";
  }
  return "BR_ERR_UNKNOWN";
}

const char* br_last_error(void) { return g_last_error.c_str(); }

const char* br_version(void) { return "blockrank-gfx950 0.1.0"; }

br_status br_attn_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                  size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_attn_plan_items(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                             int32_t* items, int64_t capacity, int64_t* n_items, int32_t* rows_per_tile) {
  return guarded([&]() -> br_status {
    if (!n_items) return record(BR_ERR_INVALID_ARG, "n_items is NULL");
    if (capacity < 0 || (capacity > 0 && !items)) return record(BR_ERR_INVALID_ARG, "items buffer is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    *n_items = int64_t(plan.items.size());
    if (rows_per_tile) *rows_per_tile = plan.rows_per_tile;
    const int64_t n = capacity < *n_items ? capacity : *n_items;
    if (n > 0) std::memcpy(items, plan.items.data(), size_t(n) * sizeof(br::AttnItem));
    return BR_OK;
  });
}

br_status br_attn_plan_schedule(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                int32_t workgroups, int32_t* sched, int64_t capacity, int32_t* ranges,
                                int64_t ranges_capacity, int64_t* n_items, int32_t* wg_per_head) {
  return guarded([&]() -> br_status {
    if (!n_items || !wg_per_head) return record(BR_ERR_INVALID_ARG, "n_items and wg_per_head must be non-NULL");
    if (workgroups < 1) return record(BR_ERR_INVALID_ARG, "workgroups must be >= 1 (got " + std::to_string(workgroups) + ")");
    if (capacity < 0 || ranges_capacity < 0) return record(BR_ERR_INVALID_ARG, "negative buffer capacity");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    br::schedule_attn_plan(dims->num_kv_heads, workgroups, &plan);
    *n_items = int64_t(plan.sched.size());
    *wg_per_head = plan.wg_per_head;
    if (sched && capacity >= *n_items && *n_items > 0)
      std::memcpy(sched, plan.sched.data(), plan.sched.size() * sizeof(br::AttnItem));
    if (ranges && ranges_capacity >= int64_t(plan.ranges.size()))
      std::memcpy(ranges, plan.ranges.data(), plan.ranges.size() * sizeof(int32_t));
    return BR_OK;
  });
}

br_status br_attn_fwd_timed(const br_dims* dims, const void* Q, const void* K, const void* V,
                            const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                            float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, workspace, workspace_bytes, stream, 0, kernel_start,
                    kernel_stop);
  });
}

br_status br_attn_routed_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                         const int32_t* keep_ptr, const int32_t* keep, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan plan;
    e = br::build_routed_plan(*dims, segment_offsets, seg_ptr, keep_ptr, keep, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_attn_routed_fwd(const br_dims* dims, const void* Q, const void* K, const void* V,
                             const int32_t* segment_offsets, const int32_t* seg_ptr, const int32_t* keep_ptr,
                             const int32_t* keep, void* out, float* lse, float softmax_scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_routed_plan(*dims, segment_offsets, seg_ptr, keep_ptr, keep, &plan);
    if (!e.ok()) return record(e);
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, workspace, workspace_bytes, stream, 0, nullptr,
                    nullptr);
  });
}

br_status br_query_attn_workspace_bytes(const br_dims* dims, int32_t corpus_len, const int32_t* query_offsets,
                                        size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan plan;
    e = br::build_query_plan(*dims, corpus_len, query_offsets, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_query_attn_fwd(const br_dims* dims, const void* Q, const void* K, const void* V, int32_t corpus_len,
                            const int32_t* query_offsets, void* out, float* lse, float softmax_scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_query_plan(*dims, corpus_len, query_offsets, &plan);
    if (!e.ok()) return record(e);
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, workspace, workspace_bytes, stream, corpus_len,
                    nullptr, nullptr);
  });
}

br_status br_attn_fwd(const br_dims* dims, const void* Q, const void* K, const void* V,
                      const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                      float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return br_attn_fwd_timed(dims, Q, K, V, segment_offsets, seg_ptr, out, lse, softmax_scale, workspace,
                           workspace_bytes, stream, nullptr, nullptr);
}

br_status br_attn_fwd_sink(const br_dims* dims, const void* Q, const void* K, const void* V,
                           const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                           float softmax_scale, float sink, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return guarded([&]() -> br_status {
    if (std::isnan(sink)) return record(BR_ERR_INVALID_ARG, "sink must not be NaN (-inf disables it)");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    const float sink_log2 = std::isinf(sink) ? sink : float(double(sink) * 1.4426950408889634);
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, workspace, workspace_bytes, stream, 0, nullptr,
                    nullptr, false, sink_log2);
  });
}

br_status br_attn_fwd_rope_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                           int32_t query_pos0, int32_t docs_after_instruction, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (docs_after_instruction != 0 && docs_after_instruction != 1)
      return record(BR_ERR_INVALID_ARG, "docs_after_instruction must be 0 or 1");
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    br::RopePlan rp;
    e = br::build_rope_plan(*dims, segment_offsets, seg_ptr, 10000.f, query_pos0, docs_after_instruction, &rp);
    if (!e.ok()) return record(e);
    RopeTable rt;
    build_rope_table(rp, dims->head_dim, plan.items.size(), &rt);
    *bytes = plan.total_bytes + rt.bytes;
    return BR_OK;
  });
}

br_status br_attn_fwd_rope(const br_dims* dims, const void* Q, const void* K, const void* V,
                           const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                           float softmax_scale, float rope_theta, int32_t query_pos0, int32_t docs_after_instruction,
                           int32_t interleaved, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (docs_after_instruction != 0 && docs_after_instruction != 1)
      return record(BR_ERR_INVALID_ARG, "docs_after_instruction must be 0 or 1");
    if (interleaved != 0 && interleaved != 1) return record(BR_ERR_INVALID_ARG, "interleaved must be 0 or 1");
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    br::AttnPlan plan;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    br::RopePlan rp;
    e = br::build_rope_plan(*dims, segment_offsets, seg_ptr, rope_theta, query_pos0, docs_after_instruction, &rp);
    if (!e.ok()) return record(e);
    return run_attn(*dims, plan, Q, K, V, out, lse, softmax_scale, workspace, workspace_bytes, stream, 0, nullptr,
                    nullptr, false, -__builtin_inff(), &rp, interleaved ? 2 : 1);
  });
}

br_status br_doc_scores_workspace_bytes(const br_dims* dims, int32_t n_signal, const int32_t* doc_offsets,
                                        const int32_t* doc_ptr, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::ScorePlan plan;
    e = br::build_score_plan(*dims, n_signal, doc_offsets, doc_ptr, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_doc_scores(const br_dims* dims, const void* Q_S, int32_t n_signal, const void* K,
                        const int32_t* doc_offsets, const int32_t* doc_ptr, float* scores, float* head_scores,
                        float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (!Q_S || !K || !scores) return record(BR_ERR_INVALID_ARG, "Q_S, K and scores must be non-NULL device pointers");
    if (!aligned(Q_S, 16) || !aligned(K, 16)) return record(BR_ERR_INVALID_ARG, "Q_S and K must be 16-byte aligned");
    if (!aligned(scores, 4) || (head_scores && !aligned(head_scores, 4)))
      return record(BR_ERR_INVALID_ARG, "scores and head_scores must be 4-byte aligned");
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
      return record(BR_ERR_INVALID_ARG, "softmax_scale must be finite");
    br::ScorePlan plan;
    e = br::build_score_plan(*dims, n_signal, doc_offsets, doc_ptr, &plan);
    if (!e.ok()) return record(e);
    if (!workspace || workspace_bytes < plan.total_bytes)
      return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_doc_scores_workspace_bytes() = " +
                                          std::to_string(plan.total_bytes));
    if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

    const int B = dims->num_prompts;
    std::vector<unsigned char> host(plan.off_ml, 0);
    std::memcpy(host.data() + plan.off_items, plan.items.data(), plan.items.size() * sizeof(br::ScoreItem));
    std::memcpy(host.data() + plan.off_doc_offsets, doc_offsets, size_t(doc_ptr[B]) * sizeof(int32_t));
    std::memcpy(host.data() + plan.off_prompt_base, plan.prompt_score_base.data(), size_t(B + 1) * sizeof(int32_t));
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    br_status st = upload(ws, host.data(), host.size(), stream);
    if (st != BR_OK) return st;

    br::ScoreLaunch a;
    a.Q_S = static_cast<const uint16_t*>(Q_S);
    a.K = static_cast<const uint16_t*>(K);
    a.items = reinterpret_cast<const br::ScoreItem*>(ws + plan.off_items);
    a.doc_offsets = reinterpret_cast<const int32_t*>(ws + plan.off_doc_offsets);
    a.prompt_base = reinterpret_cast<const int32_t*>(ws + plan.off_prompt_base);
    a.ml = reinterpret_cast<float2*>(ws + plan.off_ml);
    a.scores = scores;
    a.head_scores = head_scores;
    a.n_items = int64_t(plan.items.size());
    a.num_prompts = B;
    a.num_q_heads = dims->num_q_heads;
    a.num_kv_heads = dims->num_kv_heads;
    a.head_dim = dims->head_dim;
    a.n_signal = n_signal;
    a.row_blocks = plan.row_blocks;
    a.n_docs = plan.n_docs;
    a.scale_log2 = resolve_scale(softmax_scale, dims->head_dim) * 1.4426950408889634f;
    hipError_t he = br::launch_doc_scores(a, stream);
    if (he != hipSuccess) return hip_fail(he, "doc score kernel launch");
    return BR_OK;
  });
}

br_status br_sort_docs(const float* scores, const int32_t* doc_ptr, int32_t num_prompts, int32_t* order,
                       hipStream_t stream) {
  return guarded([&]() -> br_status {
    if (!scores || !order) return record(BR_ERR_INVALID_ARG, "scores and order must be non-NULL device pointers");
    if (!doc_ptr) return record(BR_ERR_INVALID_ARG, "doc_ptr must be a non-NULL host array");
    if (num_prompts < 1) return record(BR_ERR_INVALID_ARG, "num_prompts must be >= 1");
    if (!aligned(scores, 4) || !aligned(order, 4)) return record(BR_ERR_INVALID_ARG, "scores/order misaligned");
    std::vector<int32_t> base(size_t(num_prompts) + 1);
    for (int b = 0; b <= num_prompts; ++b) base[size_t(b)] = doc_ptr[b] - b;
    if (base[0] != 0) return record(BR_ERR_INVALID_ARG, "doc_ptr[0] must be 0");
    for (int b = 0; b < num_prompts; ++b) {
      const int32_t n = base[size_t(b) + 1] - base[size_t(b)];
      if (n < 1) return record(BR_ERR_INVALID_ARG, "prompt " + std::to_string(b) + " has no documents");
      if (n > br::kSortMaxDocs)
        return record(BR_ERR_UNSUPPORTED, "prompt " + std::to_string(b) + " has " + std::to_string(n) +
                                              " documents; at most " + std::to_string(br::kSortMaxDocs));
    }
    hipError_t he = br::launch_sort_docs(scores, base.data(), num_prompts, order, stream);
    if (he != hipSuccess) return hip_fail(he, "sort kernel launch");
    return BR_OK;
  });
}

br_status br_ssmax_softmax_scale(float s, int32_t n_docs, int32_t head_dim, float* scale) {
  return guarded([&]() -> br_status {
    if (!scale) return record(BR_ERR_INVALID_ARG, "scale is NULL");
    if (head_dim < 1) return record(BR_ERR_INVALID_ARG, "head_dim must be >= 1");
    if (n_docs < 2)
      return record(BR_ERR_INVALID_ARG, "SSMax needs n_docs >= 2 (ln 1 = 0 would make every logit zero, "
                                        "and a zero softmax_scale selects 1/sqrt(d))");
    if (!(s > 0.f) || std::isinf(s)) return record(BR_ERR_INVALID_ARG, "s must be finite and positive");
    *scale = float(double(s) * std::log(double(n_docs)) / std::sqrt(double(head_dim)));
    return BR_OK;
  });
}

br_status br_rope_workspace_bytes(const br_dims* dims, const int32_t* seg_ptr, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (!seg_ptr) return record(BR_ERR_INVALID_ARG, "seg_ptr must be a non-NULL host array");
    const int64_t runs = int64_t(seg_ptr[dims->num_prompts]) - dims->num_prompts;
    if (runs < dims->num_prompts) return record(BR_ERR_INVALID_ARG, "seg_ptr is not increasing");
    *bytes = br::rope_workspace_bytes(runs, dims->head_dim);
    return BR_OK;
  });
}


br_status br_rope_fwd(const br_dims* dims, const void* Q, const void* K, void* Q_out, void* K_out,
                      const int32_t* segment_offsets, const int32_t* seg_ptr, float rope_theta, int32_t query_pos0,
                      int32_t docs_after_instruction, int32_t interleaved, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (docs_after_instruction != 0 && docs_after_instruction != 1)
      return record(BR_ERR_INVALID_ARG, "docs_after_instruction must be 0 or 1");
    br::RopePlan plan;
    e = br::build_rope_plan(*dims, segment_offsets, seg_ptr, rope_theta, query_pos0, docs_after_instruction, &plan);
    if (!e.ok()) return record(e);
    return run_rope(*dims, seg_ptr, plan, Q, Q_out, dims->num_q_heads, K, K_out, dims->num_kv_heads, interleaved, workspace,
                    workspace_bytes, stream);
  });
}

br_status br_rope_signal_fwd(const br_dims* dims, const void* Q_S, void* Q_S_out, int32_t n_signal,
                             const int32_t* segment_offsets, const int32_t* seg_ptr, float rope_theta,
                             int32_t query_pos0, int32_t interleaved, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (!Q_S || !Q_S_out) return record(BR_ERR_INVALID_ARG, "Q_S and Q_S_out must be non-NULL device pointers");
    br::RopePlan plan;
    e = br::build_rope_signal_plan(*dims, n_signal, segment_offsets, seg_ptr, rope_theta, query_pos0, &plan);
    if (!e.ok()) return record(e);
    return run_rope(*dims, seg_ptr, plan, Q_S, Q_S_out, dims->num_q_heads, nullptr, nullptr, 0, interleaved, workspace,
                    workspace_bytes, stream);
  });
}

br_status br_rope_positions(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                            int32_t query_pos0, int32_t docs_after_instruction, int32_t* positions,
                            int64_t capacity) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (docs_after_instruction != 0 && docs_after_instruction != 1)
      return record(BR_ERR_INVALID_ARG, "docs_after_instruction must be 0 or 1");
    if (!positions) return record(BR_ERR_INVALID_ARG, "positions is NULL");
    if (capacity < dims->total_tokens)
      return record(BR_ERR_INVALID_ARG, "positions holds " + std::to_string(capacity) + " entries; need total_tokens = " +
                                            std::to_string(dims->total_tokens));
    br::RopePlan plan;
    e = br::build_rope_plan(*dims, segment_offsets, seg_ptr, 10000.f, query_pos0, docs_after_instruction, &plan);
    if (!e.ok()) return record(e);
    for (size_t r = 0; r < plan.pos0.size(); ++r)
      for (int32_t t = plan.start[r]; t < plan.start[r + 1]; ++t) positions[t] = plan.pos0[r] + (t - plan.start[r]);
    return BR_OK;
  });
}

br_status br_attn_bwd_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                      size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::BwdPlan plan;
    e = br::build_bwd_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_attn_bwd(const br_dims* dims, const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* lse, const int32_t* segment_offsets, const int32_t* seg_ptr, float* dQ, float* dK,
                      float* dV, float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV)
      return record(BR_ERR_INVALID_ARG, "Q, K, V, O, dO, lse, dQ, dK and dV must be non-NULL device pointers");
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
        !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(lse, 4))
      return record(BR_ERR_INVALID_ARG, "tensors must be 16-byte aligned (lse 4-byte)");
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
      return record(BR_ERR_INVALID_ARG, "softmax_scale must be finite");
    br::BwdPlan plan;
    e = br::build_bwd_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    if (!workspace || workspace_bytes < plan.total_bytes)
      return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_attn_bwd_workspace_bytes() = " +
                                          std::to_string(plan.total_bytes));
    if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    // Host image of the plan region: [items | merges | kv items | kv merges].
    std::vector<unsigned char> host(plan.off_part_dq, 0);
    std::memcpy(host.data() + plan.off_items, plan.fwd.items.data(), plan.fwd.items.size() * sizeof(br::AttnItem));
    if (!plan.fwd.merges.empty())
      std::memcpy(host.data() + plan.off_merges, plan.fwd.merges.data(),
                  plan.fwd.merges.size() * sizeof(br::MergeItem));
    std::memcpy(host.data() + plan.off_kv_items, plan.kv_items.data(), plan.kv_items.size() * sizeof(br::KvItem));
    if (!plan.kv_merges.empty())
      std::memcpy(host.data() + plan.off_kv_merges, plan.kv_merges.data(),
                  plan.kv_merges.size() * sizeof(br::KvMerge));
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    br_status st = upload(ws, host.data(), host.size(), stream);
    if (st != BR_OK) return st;
    br::BwdLaunch a;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.O = static_cast<const uint16_t*>(O);
    a.dO = static_cast<const uint16_t*>(dO);
    a.lse = lse;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    a.dvec = reinterpret_cast<float*>(ws + plan.off_dvec);
    a.nlse2 = a.dvec + dims->total_tokens * dims->num_q_heads;
    a.items = reinterpret_cast<const br::AttnItem*>(ws + plan.off_items);
    a.merges = reinterpret_cast<const br::MergeItem*>(ws + plan.off_merges);
    a.part_dq = reinterpret_cast<float*>(ws + plan.off_part_dq);
    a.kv_items = reinterpret_cast<const br::KvItem*>(ws + plan.off_kv_items);
    a.kv_merges = reinterpret_cast<const br::KvMerge*>(ws + plan.off_kv_merges);
    a.part_dkv = reinterpret_cast<float*>(ws + plan.off_part_dkv);
    a.n_items = int64_t(plan.fwd.items.size());
    a.n_merges = int64_t(plan.fwd.merges.size());
    a.n_kv_items = int64_t(plan.kv_items.size());
    a.n_kv_merges = int64_t(plan.kv_merges.size());
    a.total_tokens = dims->total_tokens;
    a.kv_slots = plan.kv_slots;
    a.num_q_heads = dims->num_q_heads;
    a.num_kv_heads = dims->num_kv_heads;
    a.head_dim = dims->head_dim;
    a.scale = resolve_scale(softmax_scale, dims->head_dim);
    hipError_t he = br::launch_attn_bwd(a, stream);
    if (he != hipSuccess) return hip_fail(he, "attention backward launch");
    return BR_OK;
  });
}

br_status br_attn_bwd_plan_items(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                 int32_t* items, int64_t capacity, int64_t* n_items, int32_t* n_slots) {
  return guarded([&]() -> br_status {
    if (!n_items || !n_slots) return record(BR_ERR_INVALID_ARG, "n_items and n_slots must be non-NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::BwdPlan plan;
    e = br::build_bwd_plan(*dims, segment_offsets, seg_ptr, &plan);
    if (!e.ok()) return record(e);
    *n_items = int64_t(plan.kv_items.size());
    *n_slots = plan.kv_slots;
    if (items && capacity >= *n_items)
      std::memcpy(items, plan.kv_items.data(), plan.kv_items.size() * sizeof(br::KvItem));
    return BR_OK;
  });
}

br_status br_infonce_workspace_bytes(int32_t num_prompts, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    if (num_prompts < 1) return record(BR_ERR_INVALID_ARG, "num_prompts must be >= 1");
    *bytes = br::infonce_workspace_bytes(num_prompts);
    return BR_OK;
  });
}

br_status br_infonce(const float* scores, const int32_t* doc_ptr, int32_t num_prompts, const int32_t* gold, float tau,
                     float* loss, float* dscores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return guarded([&]() -> br_status {
    if (!scores || !loss || !dscores) return record(BR_ERR_INVALID_ARG, "scores, loss and dscores must be non-NULL");
    if (!aligned(scores, 4) || !aligned(loss, 4) || !aligned(dscores, 4))
      return record(BR_ERR_INVALID_ARG, "scores, loss and dscores must be 4-byte aligned");
    br::Error e = br::validate_infonce(num_prompts, doc_ptr, gold, tau);
    if (!e.ok()) return record(e);
    const size_t need = br::infonce_workspace_bytes(num_prompts);
    if (!workspace || workspace_bytes < need)
      return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_infonce_workspace_bytes() = " +
                                          std::to_string(need));
    if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const size_t off_gold = br::align_up(size_t(num_prompts + 1) * 4, 256);
    std::vector<unsigned char> host(need, 0);
    int32_t* pb = reinterpret_cast<int32_t*>(host.data());
    for (int b = 0; b <= num_prompts; ++b) pb[b] = doc_ptr[b] - b;
    std::memcpy(host.data() + off_gold, gold, size_t(num_prompts) * 4);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    br_status st = upload(ws, host.data(), host.size(), stream);
    if (st != BR_OK) return st;
    hipError_t he = br::launch_infonce(scores, reinterpret_cast<const int32_t*>(ws),
                                       reinterpret_cast<const int32_t*>(ws + off_gold), tau, num_prompts, loss, dscores,
                                       stream);
    if (he != hipSuccess) return hip_fail(he, "InfoNCE kernel launch");
    return BR_OK;
  });
}

br_status br_doc_scores_bwd_workspace_bytes(const br_dims* dims, int32_t n_signal, const int32_t* doc_offsets,
                                            const int32_t* doc_ptr, size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::DocBwdPlan plan;
    e = br::build_doc_bwd_plan(*dims, n_signal, doc_offsets, doc_ptr, &plan);
    if (!e.ok()) return record(e);
    *bytes = plan.total_bytes;
    return BR_OK;
  });
}

br_status br_doc_scores_bwd(const br_dims* dims, const void* Q_S, int32_t n_signal, const void* K,
                            const int32_t* doc_offsets, const int32_t* doc_ptr, const float* dscores, float* dQ_S,
                            float* dK, int32_t accumulate, float softmax_scale, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    if (!Q_S || !K || !dscores || !dQ_S || !dK)
      return record(BR_ERR_INVALID_ARG, "Q_S, K, dscores, dQ_S and dK must be non-NULL device pointers");
    if (!aligned(Q_S, 16) || !aligned(K, 16) || !aligned(dQ_S, 16) || !aligned(dK, 16) || !aligned(dscores, 4))
      return record(BR_ERR_INVALID_ARG, "Q_S, K, dQ_S and dK must be 16-byte aligned (dscores 4-byte)");
    if (accumulate != 0 && accumulate != 1) return record(BR_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    if (std::isnan(softmax_scale) || std::isinf(softmax_scale))
      return record(BR_ERR_INVALID_ARG, "softmax_scale must be finite");
    br::DocBwdPlan plan;
    e = br::build_doc_bwd_plan(*dims, n_signal, doc_offsets, doc_ptr, &plan);
    if (!e.ok()) return record(e);
    if (!workspace || workspace_bytes < plan.total_bytes)
      return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_doc_scores_bwd_workspace_bytes() = " +
                                          std::to_string(plan.total_bytes));
    if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    const br::ScorePlan& sp = plan.fwd;
    const int B = dims->num_prompts;
    std::vector<unsigned char> host(sp.off_ml, 0);
    std::memcpy(host.data() + sp.off_items, sp.items.data(), sp.items.size() * sizeof(br::ScoreItem));
    std::memcpy(host.data() + sp.off_doc_offsets, doc_offsets, size_t(doc_ptr[B]) * sizeof(int32_t));
    std::memcpy(host.data() + sp.off_prompt_base, sp.prompt_score_base.data(), size_t(B + 1) * sizeof(int32_t));
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    br_status st = upload(ws, host.data(), host.size(), stream);
    if (st != BR_OK) return st;
    std::vector<int32_t> pitems((size_t(B + 1) + 3) / 4 * 4, 0);  // padded to 16 bytes
    std::copy(plan.prompt_items.begin(), plan.prompt_items.end(), pitems.begin());
    st = upload(ws + plan.off_prompt_items, pitems.data(), pitems.size() * 4, stream);
    if (st != BR_OK) return st;

    br::ScoreLaunch a;
    a.Q_S = static_cast<const uint16_t*>(Q_S);
    a.K = static_cast<const uint16_t*>(K);
    a.items = reinterpret_cast<const br::ScoreItem*>(ws + sp.off_items);
    a.doc_offsets = reinterpret_cast<const int32_t*>(ws + sp.off_doc_offsets);
    a.prompt_base = reinterpret_cast<const int32_t*>(ws + sp.off_prompt_base);
    a.ml = reinterpret_cast<float2*>(ws + sp.off_ml);
    a.scores = nullptr;
    a.head_scores = nullptr;
    a.n_items = int64_t(sp.items.size());
    a.num_prompts = B;
    a.num_q_heads = dims->num_q_heads;
    a.num_kv_heads = dims->num_kv_heads;
    a.head_dim = dims->head_dim;
    a.n_signal = n_signal;
    a.row_blocks = sp.row_blocks;
    a.n_docs = sp.n_docs;
    const float scale = resolve_scale(softmax_scale, dims->head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    hipError_t he = br::launch_doc_stats(a, stream);
    if (he != hipSuccess) return hip_fail(he, "readout statistics launch");

    br::DocBwdLaunch l;
    l.Q_S = a.Q_S;
    l.K = a.K;
    l.items = a.items;
    l.doc_offsets = a.doc_offsets;
    l.prompt_base = a.prompt_base;
    l.prompt_items = reinterpret_cast<const int32_t*>(ws + plan.off_prompt_items);
    l.ml = a.ml;
    l.rowstat = a.ml + int64_t(sp.n_docs) * n_signal * dims->num_q_heads;
    l.center = reinterpret_cast<float*>(ws + plan.off_center);
    l.dscores = dscores;
    l.dK = dK;
    l.part = reinterpret_cast<float*>(ws + plan.off_part);
    l.dQ_S = dQ_S;
    l.n_items = a.n_items;
    l.num_prompts = B;
    l.num_q_heads = dims->num_q_heads;
    l.num_kv_heads = dims->num_kv_heads;
    l.head_dim = dims->head_dim;
    l.n_signal = n_signal;
    l.row_blocks = sp.row_blocks;
    l.accumulate = accumulate;
    l.scale = scale;
    he = br::launch_doc_bwd(l, stream);
    if (he != hipSuccess) return hip_fail(he, "readout backward launch");
    return BR_OK;
  });
}

}  // extern "C"

// ---- one call for the whole hot path: attention, readout, rank ----------------------------------

namespace {

// Workspace of the fused call: [attention plan image | readout plan image | attention partials |
// readout statistics], so that both plans go up in one copy.
struct RankLayout {
  size_t score_plan = 0, attn_part = 0, score_ml = 0, total = 0;
};
RankLayout rank_layout(const br::AttnPlan& ap, const br::ScorePlan& sp) {
  RankLayout L;
  L.score_plan = br::align_up(ap.off_part_o, 256);
  L.attn_part = br::align_up(L.score_plan + sp.off_ml, 256);
  L.score_ml = br::align_up(L.attn_part + (ap.total_bytes - ap.off_part_o), 256);
  L.total = br::align_up(L.score_ml + (sp.total_bytes - sp.off_ml), 256);
  return L;
}

br_status check_sort_table(const int32_t* doc_ptr, int num_prompts, std::vector<int32_t>* base) {
  base->resize(size_t(num_prompts) + 1);
  for (int b = 0; b <= num_prompts; ++b) (*base)[size_t(b)] = doc_ptr[b] - b;
  for (int b = 0; b < num_prompts; ++b)
    if ((*base)[size_t(b) + 1] - (*base)[size_t(b)] > br::kSortMaxDocs)
      return record(BR_ERR_UNSUPPORTED, "prompt " + std::to_string(b) + " has more than " +
                                            std::to_string(br::kSortMaxDocs) + " documents to sort");
  return BR_OK;
}


// Device copy of a cached plan's upload image.  A copy of the holder (the same tables rescheduled
// for another device) starts without one.
struct DeviceImage {
  std::mutex mu;
  void* ptr = nullptr;
  DeviceImage() = default;
  DeviceImage(const DeviceImage&) {}
  DeviceImage& operator=(const DeviceImage&) = delete;
};

// Ranking-step plans, validated and scheduled, with their upload image.  Serving repeats prompt
// shapes (BlockRank pads documents to fixed chunk lengths), and planning costs about 0.15 ms per
// call at 100K tokens, so the last few plans are kept and reused when a call's dimensions and
// host tables equal an entry's element by element (and the device and its workgroup count
// match).  Entries are immutable once inserted, except for the device copy of their image, made
// once under its own mutex; a mutex guards the list.
struct RankPlan {
  int device = -1, workgroups = 0;
  br_dims dims{};
  int32_t n_signal = 0;
  std::vector<int32_t> seg_ptr, seg, doc_ptr, doc;
  br::AttnPlan ap;
  br::ScorePlan sp;
  std::vector<int32_t> base;
  RankLayout L;
  std::vector<unsigned char> host;  // the upload image
  mutable DeviceImage image;        // on `device`, from the plan's first reuse
  RankPlan() = default;
  RankPlan(const RankPlan&) = default;
  RankPlan& operator=(const RankPlan&) = delete;
  // Calls already enqueued may still read the device copy: it is freed once the device is idle
  // (if that cannot be established, it is left allocated).
  ~RankPlan() {
    if (!image.ptr) return;
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return;
    if (hipSetDevice(device) == hipSuccess && hipDeviceSynchronize() == hipSuccess) (void)hipFree(image.ptr);
    (void)hipSetDevice(cur);
  }
};

// The device copy of a cached plan's image, made at the first call that reuses the plan: a
// blocking copy followed by a device synchronisation, so that every later call, from any host
// thread or stream, reads a complete image and uploads nothing.  nullptr when the copy cannot be
// made, or while `stream` is being captured (the call then uploads into its workspace, as for a new
// plan).
const unsigned char* device_image(const RankPlan& p, hipStream_t stream) {
  std::lock_guard<std::mutex> guard(p.image.mu);
  if (!p.image.ptr) {
    // Neither the allocation nor the synchronisation may happen while the stream is captured.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
      (void)hipGetLastError();
      return nullptr;
    }
    void* d = nullptr;
    if (hipMalloc(&d, p.host.size()) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (hipMemcpy(d, p.host.data(), p.host.size(), hipMemcpyHostToDevice) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
      (void)hipGetLastError();
      (void)hipDeviceSynchronize();
      (void)hipFree(d);
      return nullptr;
    }
    p.image.ptr = d;
  }
  return static_cast<const unsigned char*>(p.image.ptr);
}

bool same_tables(const RankPlan& e, const br_dims& d, int32_t n_signal, const int32_t* so, const int32_t* sp,
                 const int32_t* dof, const int32_t* dp) {
  if (e.dims.num_prompts != d.num_prompts || e.dims.num_q_heads != d.num_q_heads ||
      e.dims.num_kv_heads != d.num_kv_heads || e.dims.head_dim != d.head_dim ||
      e.dims.total_tokens != d.total_tokens || e.n_signal != n_signal)
    return false;
  const size_t B = size_t(d.num_prompts);
  // The pointer tables first: equal to a validated entry's, they bound what the arrays hold.
  if (std::memcmp(e.seg_ptr.data(), sp, (B + 1) * sizeof(int32_t)) != 0) return false;
  if (std::memcmp(e.doc_ptr.data(), dp, (B + 1) * sizeof(int32_t)) != 0) return false;
  return std::memcmp(e.seg.data(), so, e.seg.size() * sizeof(int32_t)) == 0 &&
         std::memcmp(e.doc.data(), dof, e.doc.size() * sizeof(int32_t)) == 0;
}

class RankPlanCache {
 public:
  std::shared_ptr<const RankPlan> find(const br_dims& d, int32_t n_signal, const int32_t* so, const int32_t* sp,
                                       const int32_t* dof, const int32_t* dp) {
    std::lock_guard<std::mutex> lock(mu_);
    for (auto it = lru_.begin(); it != lru_.end(); ++it)
      if (same_tables(**it, d, n_signal, so, sp, dof, dp)) {
        auto hit = *it;
        lru_.erase(it);
        lru_.push_front(hit);
        return hit;
      }
    return nullptr;
  }
  void insert(std::shared_ptr<const RankPlan> e) {
    std::lock_guard<std::mutex> lock(mu_);
    lru_.push_front(std::move(e));
    while (lru_.size() > kEntries) lru_.pop_back();
  }

 private:
  static constexpr size_t kEntries = 4;
  std::mutex mu_;
  std::list<std::shared_ptr<const RankPlan>> lru_;
};

RankPlanCache& rank_plans() {
  static RankPlanCache* c = new RankPlanCache;  // kept until the process ends
  return *c;
}

}  // namespace

extern "C" {

br_status br_rank_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                  int32_t n_signal, const int32_t* doc_offsets, const int32_t* doc_ptr,
                                  size_t* bytes) {
  return guarded([&]() -> br_status {
    if (!bytes) return record(BR_ERR_INVALID_ARG, "bytes is NULL");
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br::AttnPlan ap;
    e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &ap);
    if (!e.ok()) return record(e);
    br::ScorePlan sp;
    e = br::build_score_plan(*dims, n_signal, doc_offsets, doc_ptr, &sp);
    if (!e.ok()) return record(e);
    *bytes = rank_layout(ap, sp).total;
    return BR_OK;
  });
}

br_status br_rank_prompts_timed(const br_dims* dims, const void* Q, const void* K, const void* V, const void* Q_S,
                                int32_t n_signal, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                const int32_t* doc_offsets, const int32_t* doc_ptr, void* out, float* lse,
                                float* scores, float* head_scores, int32_t* order, float softmax_scale,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t kernel_start, hipEvent_t kernel_stop) {
  return guarded([&]() -> br_status {
    br::Error e = br::validate_dims(dims);
    if (!e.ok()) return record(e);
    br_status st = check_attn_buffers(Q, K, V, out, lse, softmax_scale);
    if (st != BR_OK) return st;
    if (!Q_S || !scores || !order) return record(BR_ERR_INVALID_ARG, "Q_S, scores and order must be non-NULL");
    if (!aligned(Q_S, 16) || !aligned(scores, 4) || !aligned(order, 4) || (head_scores && !aligned(head_scores, 4)))
      return record(BR_ERR_INVALID_ARG, "Q_S must be 16-byte aligned; scores, head_scores and order 4-byte");
    // A cached plan for these exact tables (validated when it was made), else a new one.
    const bool tables = segment_offsets && seg_ptr && doc_offsets && doc_ptr;
    std::shared_ptr<const RankPlan> plan =
        tables ? rank_plans().find(*dims, n_signal, segment_offsets, seg_ptr, doc_offsets, doc_ptr) : nullptr;
    std::shared_ptr<RankPlan> fresh;
    if (!plan) {
      fresh = std::make_shared<RankPlan>();
      e = br::build_attn_plan(*dims, segment_offsets, seg_ptr, &fresh->ap);
      if (!e.ok()) return record(e);
      e = br::build_score_plan(*dims, n_signal, doc_offsets, doc_ptr, &fresh->sp);
      if (!e.ok()) return record(e);
      st = check_sort_table(doc_ptr, dims->num_prompts, &fresh->base);
      if (st != BR_OK) return st;
      fresh->L = rank_layout(fresh->ap, fresh->sp);
    }
    const RankLayout& L0 = plan ? plan->L : fresh->L;
    if (!workspace || workspace_bytes < L0.total)
      return record(BR_ERR_WORKSPACE, "workspace is NULL or smaller than br_rank_workspace_bytes() = " +
                                          std::to_string(L0.total));
    if (!aligned(workspace, 16)) return record(BR_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    int workgroups = 0, device = 0;
    hipError_t he = attn_workgroups(&workgroups);
    if (he == hipSuccess) he = hipGetDevice(&device);
    if (he != hipSuccess) return hip_fail(he, "device query");
    const int B = dims->num_prompts;
    if (plan && (plan->workgroups != workgroups || plan->device != device)) {
      fresh = std::make_shared<RankPlan>(*plan);  // same tables, another device: reschedule
      plan = nullptr;
    }
    if (!plan) {
      RankPlan& P = *fresh;
      br::schedule_attn_plan(dims->num_kv_heads, workgroups, &P.ap);
      P.device = device;
      P.workgroups = workgroups;
      P.dims = *dims;
      P.n_signal = n_signal;
      P.seg_ptr.assign(seg_ptr, seg_ptr + B + 1);
      P.seg.assign(segment_offsets, segment_offsets + seg_ptr[B]);
      P.doc_ptr.assign(doc_ptr, doc_ptr + B + 1);
      P.doc.assign(doc_offsets, doc_offsets + doc_ptr[B]);
      // One host image for both plans, one copy.
      const br::AttnPlan& ap = P.ap;
      const br::ScorePlan& sp = P.sp;
      P.host.assign(P.L.score_plan + sp.off_ml, 0);
      unsigned char* h = P.host.data();
      std::memcpy(h + ap.off_items, ap.sched.data(), ap.sched.size() * sizeof(br::AttnItem));
      std::memcpy(h + ap.off_ranges, ap.ranges.data(), ap.ranges.size() * sizeof(int32_t));
      if (!ap.merges.empty())
        std::memcpy(h + ap.off_merges, ap.merges.data(), ap.merges.size() * sizeof(br::MergeItem));
      unsigned char* hs = h + P.L.score_plan;
      std::memcpy(hs + sp.off_items, sp.items.data(), sp.items.size() * sizeof(br::ScoreItem));
      std::memcpy(hs + sp.off_doc_offsets, doc_offsets, size_t(doc_ptr[B]) * sizeof(int32_t));
      std::memcpy(hs + sp.off_prompt_base, sp.prompt_score_base.data(), size_t(B + 1) * sizeof(int32_t));
      rank_plans().insert(fresh);
      plan = fresh;
    }
    const br::AttnPlan& ap = plan->ap;
    const br::ScorePlan& sp = plan->sp;
    const std::vector<int32_t>& base = plan->base;
    const RankLayout& L = plan->L;
    const std::vector<unsigned char>& host = plan->host;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    // A reused plan is read from its device copy; a new one is uploaded into the workspace.
    const unsigned char* img = fresh ? nullptr : device_image(*plan, stream);
    if (!img) {
      st = upload(ws, host.data(), host.size(), stream);
      if (st != BR_OK) return st;
      img = ws;
    }

    br::AttnLaunch a;
    a.Q = static_cast<const uint16_t*>(Q);
    a.K = static_cast<const uint16_t*>(K);
    a.V = static_cast<const uint16_t*>(V);
    a.O = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.items = reinterpret_cast<const br::AttnItem*>(img + ap.off_items);
    a.ranges = reinterpret_cast<const int32_t*>(img + ap.off_ranges);
    a.merges = reinterpret_cast<const br::MergeItem*>(img + ap.off_merges);
    a.part_o = reinterpret_cast<float*>(ws + L.attn_part);
    a.part_ml = reinterpret_cast<float*>(ws + L.attn_part + (ap.off_part_ml - ap.off_part_o));
    a.n_items = int64_t(ap.items.size());
    a.n_merges = int64_t(ap.merges.size());
    a.wg_per_head = ap.wg_per_head;
    a.num_q_heads = dims->num_q_heads;
    a.num_kv_heads = dims->num_kv_heads;
    a.head_dim = dims->head_dim;
    const float scale = resolve_scale(softmax_scale, dims->head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.q_row_base = 0;
    a.ev_start = kernel_start;
    a.ev_stop = kernel_stop;

    const unsigned char* wsp = img + L.score_plan;
    br::ScoreLaunch r;
    r.Q_S = static_cast<const uint16_t*>(Q_S);
    r.K = static_cast<const uint16_t*>(K);
    r.items = reinterpret_cast<const br::ScoreItem*>(wsp + sp.off_items);
    r.doc_offsets = reinterpret_cast<const int32_t*>(wsp + sp.off_doc_offsets);
    r.prompt_base = reinterpret_cast<const int32_t*>(wsp + sp.off_prompt_base);
    r.ml = reinterpret_cast<float2*>(ws + L.score_ml);
    r.scores = scores;
    r.head_scores = head_scores;
    r.n_items = int64_t(sp.items.size());
    r.num_prompts = B;
    r.num_q_heads = dims->num_q_heads;
    r.num_kv_heads = dims->num_kv_heads;
    r.head_dim = dims->head_dim;
    r.n_signal = n_signal;
    r.row_blocks = sp.row_blocks;
    r.n_docs = sp.n_docs;
    r.scale_log2 = a.scale_log2;
    // The side stream, for large batches (if it cannot be created, the step runs on the caller's
    // stream alone).  Events around the attention kernel are recorded on the caller's stream in
    // either case, so a timed step measures the kernel as it runs in an untimed one.
    SideStream* side = nullptr;
    if (dims->total_tokens >= kSideStreamMinTokens && side_stream(&side) != hipSuccess) {
      side = nullptr;
      (void)hipGetLastError();  // clear it, so the launches below do not report it
    }
    if (!side) {
      // Everything on the caller's stream, the split-key merge in the launch of the readout's
      // partial kernel: for short batches (the fork and join cost more than the overlap saves:
      // measured at 12,864 tokens).
      a.defer_merge = true;
      he = br::launch_attn(a, stream);
      if (he != hipSuccess) return hip_fail(he, "attention kernel launch");
      he = br::launch_merge_doc_scores(a, r, stream);
      if (he != hipSuccess) return hip_fail(he, "merge and doc score kernel launch");
      he = br::launch_sort_docs(scores, base.data(), B, order, stream);
      if (he != hipSuccess) return hip_fail(he, "sort kernel launch");
      return BR_OK;
    }
    // The readout and rank read only the inputs: they run on the side stream, forked after the
    // plan upload (if any), while the attention and its merge run on the caller's stream; the caller's
    // stream then waits for them.
    std::lock_guard<std::mutex> guard(side->lock);
    he = hipEventRecord(side->fork, stream);
    if (he == hipSuccess) he = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (he != hipSuccess) return hip_fail(he, "readout fork");
    he = br::launch_attn(a, stream);  // first: it takes every CU; the readout fills its tail
    if (he != hipSuccess) return hip_fail(he, "attention kernel launch");
    he = br::launch_doc_scores(r, side->stream);
    if (he != hipSuccess) return hip_fail(he, "doc score kernel launch");
    he = br::launch_sort_docs(scores, base.data(), B, order, side->stream);
    if (he != hipSuccess) return hip_fail(he, "sort kernel launch");
    he = hipEventRecord(side->join, side->stream);
    if (he != hipSuccess) return hip_fail(he, "readout join");
    he = hipStreamWaitEvent(stream, side->join, 0);
    if (he != hipSuccess) return hip_fail(he, "readout join");
    return BR_OK;
  });
}

br_status br_rank_prompts(const br_dims* dims, const void* Q, const void* K, const void* V, const void* Q_S,
                          int32_t n_signal, const int32_t* segment_offsets, const int32_t* seg_ptr,
                          const int32_t* doc_offsets, const int32_t* doc_ptr, void* out, float* lse, float* scores,
                          float* head_scores, int32_t* order, float softmax_scale, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return br_rank_prompts_timed(dims, Q, K, V, Q_S, n_signal, segment_offsets, seg_ptr, doc_offsets, doc_ptr, out,
                               lse, scores, head_scores, order, softmax_scale, workspace, workspace_bytes, stream,
                               nullptr, nullptr);
}

}  // extern "C"
