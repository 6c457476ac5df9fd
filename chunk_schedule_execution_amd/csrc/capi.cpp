// C ABI entry points and the device runtime of a plan: upload of the lowered
// tables, plan-owned staging / scratch / flag memory, epochs, launch, status, trace.
#include <hip/hip_ext.h>
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "ccl_internal.h"

using namespace ccl;

namespace {

thread_local std::string g_detail;

int set_error(int code, const std::string& msg) {
  g_detail = msg;
  return code;
}

#define HIP_TRY(expr)                                                                        \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) fail(CCL_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

template <typename F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const Error& e) {
    return set_error(e.code, e.what());
  } catch (const std::bad_alloc&) {
    return set_error(CCL_ERR_OUT_OF_RESOURCES, "host allocation failed");
  } catch (const std::exception& e) {
    return set_error(CCL_ERR_INTERNAL, e.what());
  } catch (...) {
    return set_error(CCL_ERR_INTERNAL, "unknown exception");
  }
}

}  // namespace

struct ccl_plan {
  HostPlan hp;
  bool device = false;
  int device_id = -1;
  std::vector<void*> allocs;
  DevWG* d_wgs = nullptr;
  int32_t* d_waits = nullptr;
  unsigned long long* d_xflags = nullptr;
  unsigned long long* d_dflags = nullptr;
  unsigned char* d_staging = nullptr;
  unsigned char* d_scratch = nullptr;
  unsigned int* d_err = nullptr;
  unsigned long long* d_abort = nullptr;
  unsigned long long* d_trace = nullptr;
  unsigned long long* d_xcd = nullptr;  // per launch-grid workgroup: XCD tag of the latest launch
  void* spec_fn = nullptr;              // generated kernel (CCL_FLAG_SPECIALIZE / LAZY), or the interpreter
  int spec_shapes = 0, spec_instructions = 0, spec_waves = 0, spec_scalar_recs = 0;
  int64_t spec_code_bytes = 0;
  hipEvent_t last = nullptr;    // recorded on last_stream when another stream needs ordering
  hipStream_t last_stream = nullptr;
  bool launched = false;
  // per-count instruction geometry, least recently used replaced first
  struct GeoEntry {
    int64_t count = -1;
    DevExec* d = nullptr;
    uint64_t used = 0;
  };
  std::vector<GeoEntry> geo;
  uint64_t geo_clock = 0;
  std::vector<DevExec> geo_host;
  unsigned long long epoch = 0;
  long long timeout_ticks = 0;
  int64_t scratch_stride = 0;  // bytes between ranks' scratch
  uint64_t id = 0;             // unique per plan created in this process
  // the last ccl_execute_static launch of this plan (its state lives in the static scratch)
  bool static_launched = false;
  int static_device = -1;
  hipStream_t static_stream = nullptr;
  std::mutex mu;

  void* dev_alloc(size_t bytes) {
    void* p = nullptr;
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) fail(CCL_ERR_OUT_OF_RESOURCES, "hipMalloc(" + std::to_string(bytes) + "): " + hipGetErrorString(e));
    allocs.push_back(p);
    return p;
  }
  void release() {
    if (launched) (void)hipStreamSynchronize(last_stream);
    if (last) {
      (void)hipEventDestroy(last);
      last = nullptr;
    }
    for (void* p : allocs) (void)hipFree(p);
    allocs.clear();
  }
  ~ccl_plan() { release(); }
};

namespace {

// CCL_FLAG_DEBUG_POISON fill: every byte of the staging slots and scratch, so every
// 4-byte word (and an LL unit's flag) reads kPoisonWord.
constexpr int kPoisonByte = 0xFA;
constexpr uint32_t kPoisonWord = 0xFAFAFAFAu;

// XCD-local layout: every transfer between workgroups whose launch ids are congruent
// mod 8, which the round-robin dispatch over the eight XCDs places on one XCD (the
// kernel checks each launch's actual placement through the published tags).
bool xcd_local_layout(const HostPlan& hp) {
  bool local = !(hp.cfg.flags & CCL_FLAG_COHERENT_ONLY);
  for (size_t w = 0; w < hp.dwg.size() && local && !(hp.cfg.flags & CCL_FLAG_FORCE_XCD_LOCAL); ++w)
    for (int t = 0; t < hp.dwg[w].n && local; ++t) {
      const DevInstr& D = hp.dins[hp.dwg[w].first + t];
      if (D.peer_wg >= 0 && int(w) % 8 != D.peer_wg % 8) local = false;
    }
  return local;
}

// Argument checks shared by ccl_execute and ccl_execute_static.
void check_exec_args(const HostPlan& hp, const void* const* sendbufs, void* const* recvbufs, int64_t count) {
  if (!sendbufs || !recvbufs) fail(CCL_ERR_INVALID_ARGUMENT, "null buffer table");
  if (count < 0 || count > hp.cfg.max_count) fail(CCL_ERR_INVALID_ARGUMENT, "count out of range [0, max_count]");
  if (count % hp.granule)
    fail(CCL_ERR_INVALID_ARGUMENT, "count must be a multiple of " + std::to_string(hp.granule) + " for this program");
  for (int r = 0; r < hp.P; ++r) {
    if (!sendbufs[r] || !recvbufs[r]) fail(CCL_ERR_INVALID_ARGUMENT, "null buffer for rank " + std::to_string(r));
    if (sendbufs[r] == recvbufs[r]) fail(CCL_ERR_INVALID_ARGUMENT, "in-place execution is not supported");
  }
}

// The launch epoch is a kernel argument: a captured launch replayed from a graph would
// reuse it and find its flags already set by the previous replay. Checked before any
// other HIP call, so a capture in progress is left untouched.
void refuse_capture(void* stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cap));
  if (cap != hipStreamCaptureStatusNone)
    fail(CCL_ERR_UNSUPPORTED, "a collective launch cannot be captured into a graph (each launch needs a fresh epoch)");
}

// Next launch epoch after `e`: its low 32 bits are an LL unit's flag, so never 0 (the
// slots' initial value) nor what CCL_FLAG_DEBUG_POISON leaves in them.
unsigned long long next_epoch(unsigned long long e) {
  ++e;
  while (uint32_t(e) == 0 || uint32_t(e) == kPoisonWord) ++e;
  return e;
}

std::atomic<uint64_t> g_plan_ids{0};

// Host-side state of the static scratch on one device: the launch epoch (shared by every
// static launch there, so flags a previous launch left are always older), which plan's
// tables the array holds and for which count, and device facts looked up once.
struct StaticDevice {
  std::mutex mu;
  unsigned long long epoch = 0;
  uint64_t plan_id = 0;
  int64_t count = -1;
  int cus = 0, rate_khz = 0;
  std::vector<unsigned char> image;  // tables and records as uploaded
};
StaticDevice g_static[kMaxDevices];

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <typename T>
T* upload(ccl_plan* p, const std::vector<T>& v) {
  T* d = static_cast<T*>(p->dev_alloc(std::max<size_t>(1, v.size()) * sizeof(T)));
  if (!v.empty()) HIP_TRY(hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

void setup_device(ccl_plan* p) {
  HostPlan& hp = p->hp;
  HIP_TRY(hipGetDevice(&p->device_id));
  int cus = 0, rate_khz = 0;
  HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device_id));
  HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, p->device_id));
  // a CU budget bounds the workgroups that must be resident at once (it never raises
  // the device's own count)
  if (hp.cu_budget > 0) cus = std::min(cus, hp.cu_budget);
  int blocks = 0;
  std::string err;
  int rc = executor_max_blocks_per_cu(hp.cfg.dtype, hp.cfg.nthreads, &blocks, &err);
  if (rc) fail(rc, err);
  hp.max_resident_wgs = blocks * cus;
  // a plan that runs a generated kernel is checked against that kernel's occupancy below
  const bool generated = (hp.cfg.flags & (CCL_FLAG_SPECIALIZE | CCL_FLAG_LAZY | CCL_FLAG_SPECIALIZE_LOOP)) != 0;
  if (!generated && int(hp.dwg.size()) > hp.max_resident_wgs)
    fail(CCL_ERR_OUT_OF_RESOURCES, "plan needs " + std::to_string(hp.dwg.size()) + " co-resident workgroups, the device holds " +
                                       std::to_string(hp.max_resident_wgs) + " at " + std::to_string(hp.cfg.nthreads) +
                                       " threads");
  if (rate_khz <= 0) rate_khz = 100000;
  p->timeout_ticks = (long long)(hp.cfg.timeout_us * (rate_khz / 1000.0));
  p->d_wgs = upload(p, hp.dwg);
  p->d_waits = upload(p, hp.dwaits);
  p->geo.resize(4);
  for (auto& g : p->geo) g.d = static_cast<DevExec*>(p->dev_alloc(std::max<size_t>(1, hp.dins.size()) * sizeof(DevExec)));
  // one spare transfer flag for failure injection (CCL_FLAG_DEBUG_DROP_FLAG)
  size_t nx = hp.dxf.size() + 1;
  int nd = 0;
  for (const auto& D : hp.dins) nd = std::max(nd, D.done_flag + 1);
  const size_t xbytes = nx * 8 * kFlagStride, dbytes = size_t(std::max(1, nd)) * 8 * kFlagStride;
  p->d_xflags = static_cast<unsigned long long*>(p->dev_alloc(xbytes));
  HIP_TRY(hipMemset(p->d_xflags, 0, xbytes));
  p->d_dflags = static_cast<unsigned long long*>(p->dev_alloc(dbytes));
  HIP_TRY(hipMemset(p->d_dflags, 0, dbytes));
  p->d_staging = static_cast<unsigned char*>(p->dev_alloc(size_t(hp.staging_bytes)));
  HIP_TRY(hipMemset(p->d_staging, 0, size_t(hp.staging_bytes)));  // LL flags start at 0, never a launch's flag
  p->scratch_stride = ((hp.scratch_elems_per_rank * hp.esz) + 255) / 256 * 256;
  if (p->scratch_stride) p->d_scratch = static_cast<unsigned char*>(p->dev_alloc(size_t(p->scratch_stride) * hp.P));
  p->d_err = static_cast<unsigned int*>(p->dev_alloc(16));
  HIP_TRY(hipMemset(p->d_err, 0, 16));
  p->d_abort = static_cast<unsigned long long*>(p->dev_alloc(8));
  HIP_TRY(hipMemset(p->d_abort, 0, 8));
  const bool local = xcd_local_layout(hp);
  if (local) {
    p->d_xcd = static_cast<unsigned long long*>(p->dev_alloc(std::max<size_t>(1, hp.dwg.size()) * 8));
    HIP_TRY(hipMemset(p->d_xcd, 0, std::max<size_t>(1, hp.dwg.size()) * 8));  // no tag matches an epoch >= 1
  }
  if (hp.cfg.flags & (CCL_FLAG_SPECIALIZE | CCL_FLAG_LAZY | CCL_FLAG_SPECIALIZE_LOOP)) {
    const std::string src = specialized_source(hp, local, (hp.cfg.flags & CCL_FLAG_LAZY) != 0,
                                               (hp.cfg.flags & CCL_FLAG_SPECIALIZE_LOOP) != 0, cus, &p->spec_shapes,
                                               &p->spec_instructions, &p->spec_waves, &p->spec_scalar_recs);
    int spec_blocks = 0;
    p->spec_fn = load_specialized(src, p->device_id, hp.cfg.nthreads, &spec_blocks, &p->spec_code_bytes);
    hp.max_resident_wgs = spec_blocks * cus;
    if (int(hp.dwg.size()) > spec_blocks * cus)
      fail(CCL_ERR_OUT_OF_RESOURCES, "plan needs " + std::to_string(hp.dwg.size()) +
                                         " co-resident workgroups, the device holds " + std::to_string(spec_blocks * cus) +
                                         " of the specialized kernel");
  }
  if (hp.cfg.flags & CCL_FLAG_TRACE) {
    const size_t tb = (hp.dwg.size() + hp.dins.size()) * 32;
    p->d_trace = static_cast<unsigned long long*>(p->dev_alloc(tb));
    HIP_TRY(hipMemset(p->d_trace, 0, tb));
  }
  HIP_TRY(hipEventCreateWithFlags(&p->last, hipEventDisableTiming));
  HIP_TRY(hipDeviceSynchronize());
  p->device = true;
}

}  // namespace

extern "C" {

int ccl_version(void) { return 1; }

const char* ccl_error_string(int status) {
  switch (status) {
    case CCL_OK: return "success";
    case CCL_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CCL_ERR_INVALID_PROGRAM: return "invalid program";
    case CCL_ERR_UNSUPPORTED: return "unsupported";
    case CCL_ERR_OUT_OF_RESOURCES: return "out of resources";
    case CCL_ERR_HIP: return "HIP runtime error";
    case CCL_ERR_TIMEOUT: return "device wait timed out";
    case CCL_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* ccl_last_error_detail(void) { return g_detail.c_str(); }

int ccl_plan_create(const ccl_program_desc* prog, int nranks, int nchunks, int parallel_factor,
                    const ccl_plan_config* cfg, ccl_plan** out) {
  if (!out) return set_error(CCL_ERR_INVALID_ARGUMENT, "null output pointer");
  *out = nullptr;
  return guarded([&] {
    ccl_plan* p = new ccl_plan();
    p->id = ++g_plan_ids;
    try {
      compile_plan(p->hp, prog, nranks, nchunks, parallel_factor, cfg);
      if (!(p->hp.cfg.flags & CCL_FLAG_HOST_ONLY)) {
        setup_device(p);
      } else {
        int blocks = std::max(1, 2048 / p->hp.cfg.nthreads);
        p->hp.max_resident_wgs = blocks * p->hp.cfg.num_cus;
        if (int(p->hp.dwg.size()) > p->hp.max_resident_wgs)
          fail(CCL_ERR_OUT_OF_RESOURCES, "plan needs more co-resident workgroups than the assumed device holds");
        if (p->hp.cfg.flags & (CCL_FLAG_SPECIALIZE | CCL_FLAG_LAZY | CCL_FLAG_SPECIALIZE_LOOP)) {
          // generate and compile, load nothing
          bool local = !(p->hp.cfg.flags & CCL_FLAG_COHERENT_ONLY);
          p->spec_code_bytes = compile_specialized(specialized_source(
              p->hp, local, (p->hp.cfg.flags & CCL_FLAG_LAZY) != 0, (p->hp.cfg.flags & CCL_FLAG_SPECIALIZE_LOOP) != 0,
              p->hp.cfg.num_cus, &p->spec_shapes, &p->spec_instructions, &p->spec_waves, &p->spec_scalar_recs));
        }
      }
    } catch (...) {
      delete p;
      throw;
    }
    *out = p;
    return CCL_OK;
  });
}

int ccl_plan_destroy(ccl_plan* plan) {
  if (!plan) return CCL_OK;
  return guarded([&] {
    delete plan;
    return CCL_OK;
  });
}

int ccl_execute(ccl_plan* plan, const void* const* sendbufs, void* const* recvbufs, int64_t count, void* stream) {
  if (!plan) return set_error(CCL_ERR_INVALID_ARGUMENT, "null plan");
  return guarded([&] {
    std::lock_guard<std::mutex> lk(plan->mu);
    HostPlan& hp = plan->hp;
    if (!plan->device) fail(CCL_ERR_INVALID_ARGUMENT, "plan was created host-only");
    check_exec_args(hp, sendbufs, recvbufs, count);
    if (count == 0) return CCL_OK;
    refuse_capture(stream);
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev != plan->device_id) fail(CCL_ERR_INVALID_ARGUMENT, "plan belongs to another device");
    // geometry for this count: cached, else computed and uploaded (synchronously,
    // after the plan's previous launch, since the replaced entry may be in use)
    ccl_plan::GeoEntry* ge = nullptr;
    for (auto& g : plan->geo)
      if (g.count == count) ge = &g;
    if (!ge) {
      ge = &plan->geo[0];
      for (auto& g : plan->geo)
        if (g.used < ge->used) ge = &g;
      compute_exec_records(hp, count, plan->geo_host);
      if (plan->launched) HIP_TRY(hipStreamSynchronize(plan->last_stream));
      if (!plan->geo_host.empty())
        HIP_TRY(hipMemcpy(ge->d, plan->geo_host.data(), plan->geo_host.size() * sizeof(DevExec), hipMemcpyHostToDevice));
      ge->count = count;
    }
    ge->used = ++plan->geo_clock;
    ExecArgs A{};
    A.wgs = plan->d_wgs;
    A.recs = ge->d;
    A.waits = plan->d_waits;
    A.xflags = plan->d_xflags;
    A.dflags = plan->d_dflags;
    A.staging = plan->d_staging;
    A.err = plan->d_err;
    A.abort_word = plan->d_abort;
    A.trace = plan->d_trace;
    A.xcd_tags = plan->d_xcd;
    const unsigned long long epoch = next_epoch(plan->epoch);
    A.slice_elems = hp.slice_elems;
    A.epoch = epoch;
    A.timeout_ticks = plan->timeout_ticks;
    A.ll = (hp.cfg.flags & CCL_FLAG_LL) ? 1 : 0;
    A.ll_flag = uint32_t(epoch);
    for (int r = 0; r < hp.P; ++r) {
      A.base[CCL_BUF_INPUT][r] = const_cast<unsigned char*>(static_cast<const unsigned char*>(sendbufs[r]));
      A.base[CCL_BUF_OUTPUT][r] = static_cast<unsigned char*>(recvbufs[r]);
      A.base[CCL_BUF_SCRATCH][r] = plan->d_scratch ? plan->d_scratch + size_t(plan->scratch_stride) * r : nullptr;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // launches of one plan are serialized: on a new stream, first wait for the old one
    if (plan->launched && s != plan->last_stream) {
      HIP_TRY(hipEventRecord(plan->last, plan->last_stream));
      HIP_TRY(hipStreamWaitEvent(s, plan->last, 0));
    }
    if (hp.cfg.flags & CCL_FLAG_DEBUG_POISON) {  // stream-ordered: after the previous launch, before this one
      if (hp.staging_bytes) HIP_TRY(hipMemsetAsync(plan->d_staging, kPoisonByte, size_t(hp.staging_bytes), s));
      if (plan->d_scratch)
        HIP_TRY(hipMemsetAsync(plan->d_scratch, kPoisonByte, size_t(plan->scratch_stride) * hp.P, s));
    }
    std::string err;
    int rc = plan->spec_fn ? launch_specialized(plan->spec_fn, A, int(hp.dwg.size()), hp.cfg.nthreads, stream, &err)
                           : launch_executor(A, hp.cfg.dtype, plan->d_xcd != nullptr,
                                             (hp.cfg.flags & CCL_FLAG_STREAMING) != 0, int(hp.dwg.size()),
                                             hp.cfg.nthreads, stream, &err);
    if (rc) fail(rc, err);
    plan->epoch = epoch;
    plan->last_stream = s;
    plan->launched = true;
    return CCL_OK;
  });
}

int ccl_execute_static(ccl_plan* plan, const void* const* sendbufs, void* const* recvbufs, int64_t count,
                       void* stream) {
  if (!plan) return set_error(CCL_ERR_INVALID_ARGUMENT, "null plan");
  return guarded([&] {
    std::lock_guard<std::mutex> lk(plan->mu);
    const HostPlan& hp = plan->hp;
    check_exec_args(hp, sendbufs, recvbufs, count);
    if (count == 0) return CCL_OK;
    refuse_capture(stream);
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (plan->device && dev != plan->device_id) fail(CCL_ERR_INVALID_ARGUMENT, "plan belongs to another device");
    if (dev < 0 || dev >= kMaxDevices) fail(CCL_ERR_INVALID_ARGUMENT, "device id out of range");
    unsigned char* base = nullptr;
    std::string err;
    int rc = static_scratch_base(dev, &base, &err);
    if (rc) fail(rc, err);
    StaticDevice& st = g_static[dev];
    std::lock_guard<std::mutex> lk2(st.mu);
    if (!st.cus) {
      HIP_TRY(hipDeviceGetAttribute(&st.cus, hipDeviceAttributeMultiprocessorCount, dev));
      HIP_TRY(hipDeviceGetAttribute(&st.rate_khz, hipDeviceAttributeWallClockRate, dev));
      if (st.rate_khz <= 0) st.rate_khz = 100000;
    }
    // every workgroup of the interpreting kernel must be resident at once (within the
    // plan's CU budget)
    int blocks = 0;
    rc = executor_max_blocks_per_cu(hp.cfg.dtype, hp.cfg.nthreads, &blocks, &err);
    if (rc) fail(rc, err);
    const int cus = hp.cu_budget > 0 ? std::min(st.cus, hp.cu_budget) : st.cus;
    const size_t grid = hp.dwg.size();
    if (int64_t(grid) > int64_t(blocks) * cus)
      fail(CCL_ERR_OUT_OF_RESOURCES, "plan needs " + std::to_string(grid) + " co-resident workgroups, the device holds " +
                                         std::to_string(blocks * cus) + " of the interpreting kernel");
    // sizes against the fixed regions and the variable one
    int nd = 0;
    for (const auto& D : hp.dins) nd = std::max(nd, D.done_flag + 1);
    const size_t nx = hp.dxf.size() + 1;  // + the spare flag of CCL_FLAG_DEBUG_DROP_FLAG
    const size_t scr_stride = size_t(align256(size_t(hp.scratch_elems_per_rank * hp.esz)));
    const size_t off_wgs = kStaticVarOff;
    const size_t off_waits = align256(off_wgs + grid * sizeof(DevWG));
    const size_t off_recs = align256(off_waits + hp.dwaits.size() * 4);
    const size_t off_stage = align256(off_recs + hp.dins.size() * sizeof(DevExec));
    const size_t off_scr = align256(off_stage + size_t(hp.staging_bytes));
    const size_t end = off_scr + scr_stride * hp.P;
    if (nx * 8 * kFlagStride > kStaticXflagBytes || size_t(nd) * 8 * kFlagStride > kStaticDflagBytes ||
        grid * 8 > kStaticTagBytes || end > kStaticScratchBytes)
      fail(CCL_ERR_OUT_OF_RESOURCES,
           "plan needs " + std::to_string(end) + " bytes of the static scratch (at most " +
               std::to_string(kStaticScratchBytes) + "), " + std::to_string(nx) + " transfer flags (at most " +
               std::to_string(kStaticXflagBytes / (8 * kFlagStride)) + "), " + std::to_string(nd) +
               " completion flags (at most " + std::to_string(kStaticDflagBytes / (8 * kFlagStride)) + ") and " +
               std::to_string(grid) + " workgroups (at most " + std::to_string(kStaticTagBytes / 8) + ")");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // tables and records for this plan and count, unless the array holds them already
    // (stream-ordered after every earlier launch on this stream; the host image stays
    // valid until the copy has completed)
    if (st.plan_id != plan->id || st.count != count) {
      std::vector<DevExec> recs;
      compute_exec_records(hp, count, recs);
      st.image.assign(off_stage - off_wgs, 0);
      std::memcpy(st.image.data(), hp.dwg.data(), grid * sizeof(DevWG));
      if (!hp.dwaits.empty()) std::memcpy(st.image.data() + (off_waits - off_wgs), hp.dwaits.data(), hp.dwaits.size() * 4);
      if (!recs.empty()) std::memcpy(st.image.data() + (off_recs - off_wgs), recs.data(), recs.size() * sizeof(DevExec));
      HIP_TRY(hipMemcpyAsync(base + off_wgs, st.image.data(), st.image.size(), hipMemcpyHostToDevice, s));
      HIP_TRY(hipStreamSynchronize(s));
      st.plan_id = plan->id;
      st.count = count;
    }
    // clear what must start at zero: the error word, and low-latency slots (their flag
    // words must never hold this launch's flag); poison mode fills slots and scratch
    HIP_TRY(hipMemsetAsync(base + kStaticErrOff, 0, 16, s));
    const bool ll = (hp.cfg.flags & CCL_FLAG_LL) != 0;
    if (hp.cfg.flags & CCL_FLAG_DEBUG_POISON) {
      if (hp.staging_bytes) HIP_TRY(hipMemsetAsync(base + off_stage, kPoisonByte, size_t(hp.staging_bytes), s));
      if (scr_stride) HIP_TRY(hipMemsetAsync(base + off_scr, kPoisonByte, scr_stride * hp.P, s));
    } else if (ll && hp.staging_bytes) {
      HIP_TRY(hipMemsetAsync(base + off_stage, 0, size_t(hp.staging_bytes), s));
    }
    const bool local = xcd_local_layout(hp);
    const unsigned long long epoch = next_epoch(st.epoch);
    ExecArgs A{};
    A.wgs = reinterpret_cast<const DevWG*>(base + off_wgs);
    A.recs = reinterpret_cast<const DevExec*>(base + off_recs);
    A.waits = reinterpret_cast<const int32_t*>(base + off_waits);
    A.xflags = reinterpret_cast<unsigned long long*>(base + kStaticXflagOff);
    A.dflags = reinterpret_cast<unsigned long long*>(base + kStaticDflagOff);
    A.staging = base + off_stage;
    A.err = reinterpret_cast<unsigned int*>(base + kStaticErrOff);
    A.abort_word = reinterpret_cast<unsigned long long*>(base + kStaticErrOff + 16);
    A.trace = nullptr;
    A.xcd_tags = local ? reinterpret_cast<unsigned long long*>(base + kStaticTagOff) : nullptr;
    A.slice_elems = hp.slice_elems;
    A.epoch = epoch;
    A.timeout_ticks = (long long)(hp.cfg.timeout_us * (st.rate_khz / 1000.0));
    A.ll = ll ? 1 : 0;
    A.ll_flag = uint32_t(epoch);
    for (int r = 0; r < hp.P; ++r) {
      A.base[CCL_BUF_INPUT][r] = const_cast<unsigned char*>(static_cast<const unsigned char*>(sendbufs[r]));
      A.base[CCL_BUF_OUTPUT][r] = static_cast<unsigned char*>(recvbufs[r]);
      A.base[CCL_BUF_SCRATCH][r] = scr_stride ? base + off_scr + scr_stride * r : nullptr;
    }
    rc = launch_executor(A, hp.cfg.dtype, local, (hp.cfg.flags & CCL_FLAG_STREAMING) != 0, int(grid),
                         hp.cfg.nthreads, stream, &err);
    if (rc) fail(rc, err);
    st.epoch = epoch;
    plan->static_launched = true;
    plan->static_device = dev;
    plan->static_stream = s;
    return CCL_OK;
  });
}

int ccl_plan_info(const ccl_plan* plan, ccl_plan_info_t* info) {
  if (!plan || !info) return set_error(CCL_ERR_INVALID_ARGUMENT, "null argument");
  return guarded([&] {
    const HostPlan& hp = plan->hp;
    std::memset(info, 0, sizeof *info);
    info->nranks = hp.P;
    info->nchunks = hp.C;
    info->parallel_factor = hp.k;
    info->dtype = hp.cfg.dtype;
    info->num_workgroups = 0;
    for (const auto& G : hp.dwg) info->num_workgroups += G.n > 0 ? 1 : 0;
    info->grid_workgroups = int(hp.dwg.size());
    info->xcd_local = plan->d_xcd ? 1 : 0;
    info->specialized_shapes = plan->spec_shapes;
    info->specialized_instructions = plan->spec_instructions;
    info->specialized_waves_per_simd = plan->spec_waves;
    info->specialized_code_bytes = plan->spec_code_bytes;
    info->max_wg_per_rank = hp.max_wg_per_rank;
    info->num_instructions = int(hp.dins.size());
    info->num_subpipelines = hp.num_subpipes;
    info->num_connections = hp.num_connections;
    info->num_transfers = int(hp.dxf.size());
    info->num_waits = int(hp.dwaits.size());
    info->count_granule = hp.granule;
    info->nthreads = hp.cfg.nthreads;
    info->slice_bytes = int(hp.slice_elems * hp.esz);
    info->max_resident_wgs = hp.max_resident_wgs;
    info->staging_bytes = hp.staging_bytes;
    info->scratch_bytes = hp.scratch_elems_per_rank * hp.esz * hp.P;
    int nd = 0;
    for (const auto& D : hp.dins) nd = std::max(nd, D.done_flag + 1);
    info->flag_bytes = int64_t(hp.dxf.size() + nd) * 8 * kFlagStride;
    info->table_bytes = int64_t(hp.dwg.size() * sizeof(DevWG) + hp.dins.size() * sizeof(DevExec) * 4 +
                                hp.dwaits.size() * 4);
    for (int i = 0; i < 6; ++i) info->compile_ms[i] = hp.ms[i];
    for (const auto& D : hp.dins) info->opcode_hist[D.op & 15]++;
    info->dag_width = hp.dag_width;
    info->dag_depth = hp.dag_depth;
    info->specialized_scalar_records = plan->spec_scalar_recs;
    return CCL_OK;
  });
}

int64_t ccl_plan_bytes(const ccl_plan* plan, int64_t count) {
  if (!plan) return set_error(CCL_ERR_INVALID_ARGUMENT, "null plan");
  if (count < 0 || count > plan->hp.cfg.max_count) return set_error(CCL_ERR_INVALID_ARGUMENT, "count out of range");
  int64_t v = 0;
  int rc = guarded([&] {
    v = plan_bytes(plan->hp, count);
    return CCL_OK;
  });
  return rc ? rc : v;
}

int ccl_plan_export(const ccl_plan* plan, ccl_instr_info* out, size_t cap, size_t* n) {
  if (!plan || !n || (cap && !out)) return set_error(CCL_ERR_INVALID_ARGUMENT, "null argument");
  return guarded([&] {
    const HostPlan& hp = plan->hp;
    *n = hp.dins.size();
    size_t j = 0;
    for (size_t w = 0; w < hp.dwg.size(); ++w) {
      const DevWG& G = hp.dwg[w];
      for (int t = 0; t < G.n && j < cap; ++t, ++j) {
        const DevInstr& D = hp.dins[G.first + t];
        const Instr& I = hp.ins[hp.dins_base[G.first + t]];
        ccl_instr_info& o = out[j];
        o.rank = G.rank;
        o.wg = int(w);
        o.subpipe = I.sp;
        o.channel = I.channel;
        o.instance = D.instance;
        o.opcode = int(D.op);
        o.a_buf = D.a_buf;
        o.a_idx = D.a_idx;
        o.b_buf = D.b_buf;
        o.b_idx = D.b_idx;
        o.d_buf = D.d_buf;
        o.d_idx = D.d_idx;
        o.count = D.cnt;
        o.recv_peer = I.xin >= 0 ? hp.xf[I.xin].src_rank : -1;
        o.send_peer = I.xout >= 0 ? hp.xf[I.xout].dst_rank : -1;
        o.xin = D.xin;
        o.xout = D.xout;
        o.nwaits = D.nwaits;
        o.chunk_id = I.chunk_id;
        o.done_flag = D.done_flag;
      }
    }
    return CCL_OK;
  });
}

int ccl_plan_check(const ccl_plan* plan, uint64_t seed, int nsims) {
  if (!plan || nsims < 0) return set_error(CCL_ERR_INVALID_ARGUMENT, "bad argument");
  return guarded([&] {
    check_lowered(plan->hp, seed, nsims);
    return CCL_OK;
  });
}

int ccl_plan_status(ccl_plan* plan) {
  if (!plan) return set_error(CCL_ERR_INVALID_ARGUMENT, "null plan");
  return guarded([&] {
    std::lock_guard<std::mutex> lk(plan->mu);
    if (plan->static_launched) {  // the last static launch on its device reported through the static error word
      plan->static_launched = false;
      HIP_TRY(hipStreamSynchronize(plan->static_stream));
      unsigned char* base = nullptr;
      std::string err;
      int rc = static_scratch_base(plan->static_device, &base, &err);
      if (rc) fail(rc, err);
      unsigned int e[4] = {0, 0, 0, 0};
      HIP_TRY(hipMemcpy(e, base + kStaticErrOff, sizeof e, hipMemcpyDeviceToHost));
      if (e[0] != 0) {
        HIP_TRY(hipMemset(base + kStaticErrOff, 0, sizeof e));
        fail(-int(e[0]), "static launch " + std::to_string(e[3]) + ": workgroup " + std::to_string(e[1]) +
                             " timed out at instruction " + std::to_string(e[2]));
      }
    }
    if (!plan->device) return CCL_OK;
    if (plan->launched) HIP_TRY(hipStreamSynchronize(plan->last_stream));
    unsigned int e[4] = {0, 0, 0, 0};
    HIP_TRY(hipMemcpy(e, plan->d_err, sizeof e, hipMemcpyDeviceToHost));
    if (e[0] == 0) return CCL_OK;
    HIP_TRY(hipMemset(plan->d_err, 0, sizeof e));
    fail(-int(e[0]), "launch " + std::to_string(e[3]) + ": workgroup " + std::to_string(e[1]) + " timed out at instruction " +
                         std::to_string(e[2]));
  });
}

int ccl_plan_read_trace(ccl_plan* plan, void* host, size_t bytes) {
  if (!plan || !host) return set_error(CCL_ERR_INVALID_ARGUMENT, "null argument");
  return guarded([&] {
    std::lock_guard<std::mutex> lk(plan->mu);
    if (!plan->d_trace) fail(CCL_ERR_INVALID_ARGUMENT, "plan was not created with CCL_FLAG_TRACE");
    size_t need = plan->hp.dwg.size() * 32;
    if (bytes < need) fail(CCL_ERR_INVALID_ARGUMENT, "trace buffer too small");
    const size_t full = (plan->hp.dwg.size() + plan->hp.dins.size()) * 32;
    if (bytes >= full) need = full;
    if (plan->launched) HIP_TRY(hipStreamSynchronize(plan->last_stream));
    HIP_TRY(hipMemcpy(host, plan->d_trace, need, hipMemcpyDeviceToHost));
    return CCL_OK;
  });
}

int ccl_plan_link_busy(ccl_plan* plan, ccl_link_busy* out, size_t cap, size_t* n) {
  if (!plan || !n || (cap && !out)) return set_error(CCL_ERR_INVALID_ARGUMENT, "null argument");
  return guarded([&] {
    std::lock_guard<std::mutex> lk(plan->mu);
    const HostPlan& hp = plan->hp;
    if (!plan->d_trace) fail(CCL_ERR_INVALID_ARGUMENT, "plan was not created with CCL_FLAG_TRACE");
    if (!plan->launched) fail(CCL_ERR_INVALID_ARGUMENT, "the plan has not been launched");
    const size_t nwg = hp.dwg.size(), nin = hp.dins.size();
    std::vector<unsigned long long> t((nwg + nin) * 4);
    HIP_TRY(hipStreamSynchronize(plan->last_stream));
    HIP_TRY(hipMemcpy(t.data(), plan->d_trace, t.size() * 8, hipMemcpyDeviceToHost));
    unsigned long long t0 = ~0ull, t1 = 0;
    for (size_t w = 0; w < nwg; ++w)
      if (t[4 * w + 3] > 0) {  // workgroups that ran instructions
        t0 = std::min(t0, t[4 * w]);
        t1 = std::max(t1, t[4 * w + 1]);
      }
    // per connection: the intervals of the instructions that send on it
    std::map<std::array<int, 4>, std::vector<std::pair<unsigned long long, unsigned long long>>> busy;
    for (size_t w = 0; w < nwg; ++w) {
      const DevWG& G = hp.dwg[w];
      for (int j = 0; j < G.n; ++j) {
        const size_t gi = size_t(G.first + j);
        const DevInstr& D = hp.dins[gi];
        if (D.xout < 0) continue;
        const Instr& I = hp.ins[hp.dins_base[gi]];
        const Xfer& X = hp.xf[I.xout];
        const unsigned long long* r = &t[4 * (nwg + gi)];
        auto& v = busy[{X.src_rank, X.dst_rank, X.channel, D.instance}];
        if (r[0] > 0 && r[2] >= r[0]) v.emplace_back(r[0], r[2]);
      }
    }
    *n = busy.size();
    size_t j = 0;
    const double span = t1 > t0 ? double(t1 - t0) : 0.0;
    for (auto& kv : busy) {
      if (j >= cap) break;
      auto& v = kv.second;
      std::sort(v.begin(), v.end());
      unsigned long long covered = 0, lo = 0, hi = 0;
      bool open = false;
      for (const auto& iv : v) {
        if (!open || iv.first > hi) {
          if (open) covered += hi - lo;
          lo = iv.first;
          hi = iv.second;
          open = true;
        } else {
          hi = std::max(hi, iv.second);
        }
      }
      if (open) covered += hi - lo;
      out[j].src_rank = kv.first[0];
      out[j].dst_rank = kv.first[1];
      out[j].channel = kv.first[2];
      out[j].instance = kv.first[3];
      out[j].busy_fraction = span > 0 ? double(covered) / span : 0.0;
      ++j;
    }
    return CCL_OK;
  });
}

int ccl_litmus_message_passing(int cross_xcd, int rounds, int words, int64_t timeout_us, int64_t* results,
                               void* stream) {
  if (!results || rounds < 1 || rounds > 1000000 || words < 4 || words > (1 << 20) || words % 4 || timeout_us < 1)
    return set_error(CCL_ERR_INVALID_ARGUMENT, "litmus: bad arguments");
  return guarded([&] {
    constexpr int npairs = 8;  // producers 0..7; consumers 8..15 (ids congruent mod 8 share an XCD)
    const size_t region = (size_t(words) * 4 + 255) / 256 * 256;
    const size_t flag_bytes = size_t(npairs) * kFlagStride * 8;
    const size_t sizes[6] = {region * npairs, flag_bytes, flag_bytes, 2 * npairs * 8, npairs * 8 * 8, 8};
    void* bufs[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    struct Free {
      void** b;
      ~Free() {
        for (int i = 0; i < 6; ++i)
          if (b[i]) (void)hipFree(b[i]);
      }
    } guard{bufs};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int i = 0; i < 6; ++i) {
      HIP_TRY(hipMalloc(&bufs[i], sizes[i]));
      HIP_TRY(hipMemsetAsync(bufs[i], 0, sizes[i], s));
    }
    int dev = 0, rate_khz = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev));
    if (rate_khz <= 0) rate_khz = 100000;
    std::string err;
    int rc = launch_litmus_mp(static_cast<unsigned char*>(bufs[0]), static_cast<unsigned long long*>(bufs[1]),
                              static_cast<unsigned long long*>(bufs[2]), static_cast<unsigned long long*>(bufs[3]),
                              static_cast<long long*>(bufs[4]), static_cast<unsigned long long*>(bufs[5]), npairs,
                              rounds, words, cross_xcd ? 1 : 0, (long long)(timeout_us * (rate_khz / 1000.0)), stream,
                              &err);
    if (rc) fail(rc, err);
    HIP_TRY(hipStreamSynchronize(s));
    HIP_TRY(hipMemcpy(results, bufs[4], npairs * 8 * 8, hipMemcpyDeviceToHost));
    return CCL_OK;
  });
}

int ccl_hop_probe(int hops, int bytes, int two_operands, int ll, int nthreads, int launches, int64_t window_bytes,
                  int64_t timeout_us, double* us_per_hop, int64_t* info, void* stream) {
  // a hand-off region holds the payload, or under LL its units (twice the payload)
  const int64_t slot_bytes = (ll ? 2 : 1) * ((int64_t(bytes) + 255) / 256 * 256);
  if (!us_per_hop || !info || hops < 1 || hops > 31 || bytes < 16 || bytes > (4 << 20) || bytes % 16 ||
      nthreads < 64 || nthreads > 1024 || nthreads % 64 || launches < 1 || launches > 1000 || timeout_us < 1 ||
      window_bytes < 0 || window_bytes > (int64_t(16) << 20) || (window_bytes > 0 && window_bytes < 2 * slot_bytes))
    return set_error(CCL_ERR_INVALID_ARGUMENT, "hop probe: bad arguments");
  return guarded([&] {
    const size_t rbytes = size_t(slot_bytes);
    // region stride: one hand-off region, or a window the launches step through
    const size_t region = window_bytes > 0 ? std::max(rbytes, size_t(window_bytes) / 256 * 256) : rbytes;
    const int chain = hops + 1;
    // data (source + one region per chain workgroup), second operands, flags, tags,
    // ticks, watchdog words, abort word
    const size_t sizes[7] = {region * (chain + 1), region * chain, size_t(chain) * kFlagStride * 8, size_t(chain) * 8,
                             16, 16, 8};
    void* bufs[7] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    struct Free {
      void** b;
      ~Free() {
        for (int i = 0; i < 7; ++i)
          if (b[i]) (void)hipFree(b[i]);
      }
    } guard{bufs};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int i = 0; i < 7; ++i) {
      HIP_TRY(hipMalloc(&bufs[i], sizes[i]));
      HIP_TRY(hipMemsetAsync(bufs[i], 0, sizes[i], s));
    }
    int dev = 0, rate_khz = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev));
    if (rate_khz <= 0) rate_khz = 100000;
    const long long timeout_ticks = (long long)(timeout_us * (rate_khz / 1000.0));
    auto* data = static_cast<unsigned char*>(bufs[0]);
    std::vector<uint32_t> last(bytes / 4);
    std::vector<unsigned long long> tags(chain);
    for (int i = 0; i < 4; ++i) info[i] = 0;
    for (int l = 0; l < launches; ++l) {
      const unsigned long long epoch = (unsigned long long)l + 1;
      // every launch moves one payload further through the window (256-byte aligned)
      const size_t rot = region > rbytes ? (size_t(l) * rbytes) % (region - rbytes) / 256 * 256 : 0;
      const uint32_t word = 0x3f800000u + uint32_t(epoch & 0x7fffffu);  // a normal float, new every launch
      HIP_TRY(hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(data + rot), int(word), bytes / 4, s));
      std::string err;
      const int rc = launch_hop_probe(data, static_cast<unsigned char*>(bufs[1]),
                                      static_cast<unsigned long long*>(bufs[2]), static_cast<unsigned long long*>(bufs[3]),
                                      static_cast<long long*>(bufs[4]), static_cast<unsigned int*>(bufs[5]),
                                      static_cast<unsigned long long*>(bufs[6]), epoch, timeout_ticks, region, rot,
                                      hops, bytes, two_operands ? 1 : 0, ll ? 1 : 0, nthreads, stream, &err);
      if (rc) fail(rc, err);
      HIP_TRY(hipStreamSynchronize(s));
      unsigned int werr[4];
      long long ticks[2];
      HIP_TRY(hipMemcpy(werr, bufs[5], sizeof werr, hipMemcpyDeviceToHost));
      if (werr[0] != 0) {  // a wait expired: the chain stopped, and so does the probe
        info[1] += 1;
        break;
      }
      HIP_TRY(hipMemcpy(ticks, bufs[4], sizeof ticks, hipMemcpyDeviceToHost));
      HIP_TRY(hipMemcpy(tags.data(), bufs[3], tags.size() * 8, hipMemcpyDeviceToHost));
      HIP_TRY(hipMemcpy(last.data(), data + size_t(chain) * region + rot, size_t(bytes), hipMemcpyDeviceToHost));
      for (int j = 1; j < chain; ++j) info[0] += (tags[j] & 15ull) != (tags[0] & 15ull);
      for (uint32_t v : last)
        if (v != word) {
          info[2] += 1;
          break;
        }
      us_per_hop[l] = double(ticks[1] - ticks[0]) / (rate_khz / 1000.0) / hops;
      info[3] += 1;
    }
    return CCL_OK;
  });
}

int ccl_stream_create_cu_masked(const uint32_t* mask, int nwords, void** stream) {
  if (!stream) return set_error(CCL_ERR_INVALID_ARGUMENT, "null stream pointer");
  *stream = nullptr;
  if (!mask || nwords < 1 || nwords > 64) return set_error(CCL_ERR_INVALID_ARGUMENT, "mask: 1..64 32-bit words");
  return guarded([&] {
    int dev = 0, cus = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    // the runtime is handed exactly the words that cover the device's CUs (a copy the
    // size of its argument), so it never reads past the caller's array
    std::vector<uint32_t> m(mask, mask + std::min(nwords, (cus + 31) / 32));
    int set = 0;
    for (int i = 0; i < nwords * 32 && i < cus; ++i) set += (m[i / 32] >> (i % 32)) & 1u;
    if (set == 0) fail(CCL_ERR_INVALID_ARGUMENT, "the mask enables no compute unit of the device");
    hipStream_t s = nullptr;
    HIP_TRY(hipExtStreamCreateWithCUMask(&s, uint32_t(m.size()), m.data()));
    *stream = s;
    return CCL_OK;
  });
}

int ccl_stream_destroy(void* stream) {
  if (!stream) return CCL_OK;
  return guarded([&] {
    HIP_TRY(hipStreamDestroy(reinterpret_cast<hipStream_t>(stream)));
    return CCL_OK;
  });
}

int ccl_cu_probe(void* stream, int nblocks, int hold_us, uint32_t* out) {
  if (!out || nblocks < 1 || nblocks > 65536 || hold_us < 0 || hold_us > 100000)
    return set_error(CCL_ERR_INVALID_ARGUMENT, "placement probe: bad arguments");
  return guarded([&] {
    int dev = 0, rate_khz = 0;
    HIP_TRY(hipGetDevice(&dev));
    HIP_TRY(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev));
    if (rate_khz <= 0) rate_khz = 100000;
    unsigned* d = nullptr;
    const size_t bytes = size_t(nblocks) * 2 * sizeof(unsigned);
    HIP_TRY(hipMalloc(&d, bytes));
    struct Free {
      unsigned* p;
      ~Free() { (void)hipFree(p); }
    } guard{d};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    HIP_TRY(hipMemsetAsync(d, 0xFF, bytes, s));
    std::string err;
    const int rc = launch_cu_probe(d, nblocks, (long long)hold_us * (rate_khz / 1000), stream, &err);
    if (rc) fail(rc, err);
    HIP_TRY(hipStreamSynchronize(s));
    HIP_TRY(hipMemcpy(out, d, bytes, hipMemcpyDeviceToHost));
    return CCL_OK;
  });
}

int ccl_copy_probe(void* dst, const void* src, size_t bytes, int nblocks, int nthreads, void* stream) {
  if (!dst || !src || bytes % 16 || nblocks < 1 || nthreads < 64 || nthreads > 1024 || nthreads % 64)
    return set_error(CCL_ERR_INVALID_ARGUMENT, "copy probe: bad arguments");
  return guarded([&] {
    std::string err;
    int rc = launch_copy_probe(dst, src, bytes, nblocks, nthreads, stream, &err);
    if (rc) fail(rc, err);
    return CCL_OK;
  });
}

}  // extern "C"
