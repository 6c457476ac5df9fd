// Hop-latency probe for gfx950: one hand-off of the executor, timed in isolation (a
// diagnostic beside the executor, like the copy probe and the litmus test).
//
// A ring collective over P ranks is a chain of 2(P - 1) dependent hand-offs (MSCCLang
// report, section 3.1: each receive-reduce-send step waits for the previous rank's
// send); when every piece is small the launch is as long as that chain. This kernel
// builds such a chain out of separate workgroups and times it, so the executor's
// latency-bound launches can be set against the cost of the hand-offs they are made of.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/ccl.h"
#include "device_abi.h"
#include "executor_device.h"

namespace ccl {
namespace {

// Hop-latency probe: the cost of one hand-off of the executor, in isolation. A chain
// of hops + 1 workgroups on one XCD (ids 0, 8, 16, ...: ids congruent mod 8 share an
// XCD under the round-robin dispatch; the others exit at once) passes a payload along:
// workgroup 0 copies the source into region 1; workgroup j >= 1 runs the executor's
// own slice code (run_slice: one thread polls the flag, the workgroup loads region j
// with agent-coherent loads, adds the second operand if asked, stores region j + 1 with
// the XCD-local plain stores), waits for its stores and sets its flag as every send
// does. The last workgroup records the wall clock once its stores are acknowledged;
// workgroup 0 records it just before its flag store, so the difference is `hops` full
// hand-offs: flag store, flag seen, loads, stores, acknowledgements.
struct HopArgs {
  unsigned char* data;        // hops + 2 regions (stride `region`, 256-byte aligned): source, hand-offs, result
  unsigned char* second;      // per chain workgroup a region of zeros: the second operand of a reducing hop
  unsigned long long* flags;  // per chain workgroup, kFlagStride apart
  unsigned long long* tags;   // per chain workgroup: epoch << 8 | 0x10 | XCD id
  long long* ticks;           // [0] start, [1] end of this launch
  unsigned int* err;          // the watchdog's record (4 words)
  unsigned long long* abort_word;
  unsigned long long epoch;
  long long timeout_ticks;
  size_t region;  // region stride
  size_t rot;     // this launch's offset inside every region
  int hops, bytes, two_operands;
  int ll;  // low-latency protocol: regions 1..hops hold {4 data bytes, 4-byte flag} units
};

__device__ bool hop_wait_tag(unsigned long long* p, const HopArgs& A, unsigned long long& v) {
  const long long t0 = wall_clock64();
  for (unsigned it = 0;; ++it) {
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((v >> 8) == A.epoch) return true;
    if ((it & 15) == 15) {
      if (__hip_atomic_load(A.abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == A.epoch) return false;
      if (wall_clock64() - t0 > A.timeout_ticks) {
        ll_give_up_slow(A.err, A.abort_word, A.epoch, -1, -1, t0);  // records the expiry and stops the chain
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The same chain under the low-latency protocol: workgroup 0 turns the source into
// flagged units, every later workgroup polls the units it consumes, adds the second
// operand if asked and writes units for the next one (run_ll, as an LL instruction does;
// a receiver on another XCD gets the L2 written back first), and the last workgroup
// writes plain data. Workgroup 0 records the wall clock as it starts, the last one once
// its stores are acknowledged.
__device__ void hop_probe_ll(const HopArgs& A, int j, int tid, int nthr, bool colocated, const unsigned char* in,
                             const unsigned char* second, unsigned char* out, int* s_gave_up) {
  const int n = A.bytes / 4;
  const uint32_t flag = uint32_t(A.epoch);
  bool gave_up = false;
  if (j == 0) {
    if (tid == 0) A.ticks[0] = wall_clock64();
    gave_up = run_ll<CCL_F32, false, false, false, true, true>(in, in, nullptr, out, n, tid, nthr, flag, A.err,
                                                               A.abort_word, A.epoch, A.timeout_ticks, 0);
  } else if (j < A.hops) {
    gave_up = A.two_operands
                  ? run_ll<CCL_F32, true, true, false, true, true>(in, second, nullptr, out, n, tid, nthr, flag, A.err,
                                                                   A.abort_word, A.epoch, A.timeout_ticks, j)
                  : run_ll<CCL_F32, true, false, false, true, true>(in, in, nullptr, out, n, tid, nthr, flag, A.err,
                                                                    A.abort_word, A.epoch, A.timeout_ticks, j);
  } else {
    gave_up = A.two_operands
                  ? run_ll<CCL_F32, true, true, true, false, true>(in, second, out, nullptr, n, tid, nthr, flag, A.err,
                                                                   A.abort_word, A.epoch, A.timeout_ticks, j)
                  : run_ll<CCL_F32, true, false, true, false, true>(in, in, out, nullptr, n, tid, nthr, flag, A.err,
                                                                    A.abort_word, A.epoch, A.timeout_ticks, j);
  }
  if (gave_up) *s_gave_up = 1;
  if (j == A.hops || !colocated) wait_vm_stores();
  __syncthreads();
  if (*s_gave_up) return;  // the whole workgroup leaves together
  if (tid == 0) {
    if (j < A.hops && !colocated) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (j == A.hops) A.ticks[1] = wall_clock64();
  }
}

__global__ __launch_bounds__(1024) void hop_probe_kernel(HopArgs A) {
  __shared__ int s_go, s_gave_up;
  __shared__ unsigned long long s_next;
  if (blockIdx.x % 8 != 0) return;
  const int j = blockIdx.x / 8, tid = threadIdx.x, nthr = blockDim.x;
  const unsigned long long my_tag = (A.epoch << 8) | 0x10ull | xcd_id();
  if (tid == 0) {
    __hip_atomic_store(&A.tags[j], my_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_next = 0;
    s_gave_up = 0;
    s_go = j == A.hops || hop_wait_tag(&A.tags[j + 1], A, s_next);
  }
  __syncthreads();
  if (!s_go) return;
  const bool colocated = j < A.hops && s_next == my_tag;
  const unsigned char* in = A.data + size_t(j) * A.region + A.rot;
  const unsigned char* second = A.second + size_t(j) * A.region + A.rot;
  unsigned char* out = A.data + size_t(j + 1) * A.region + A.rot;
  if (A.ll) {
    hop_probe_ll(A, j, tid, nthr, colocated, in, second, out, &s_gave_up);
    return;
  }
  const int n = A.bytes / 4;
  long long waited = 0;
  if (j == 0)
    waited = run_slice<CCL_F32, false, false, false, true, true, false, false>(
        in, in, nullptr, out, n, tid, nthr, nullptr, 0, A.err, A.abort_word, A.epoch, A.timeout_ticks, 0);
  else if (A.two_operands)
    waited = run_slice<CCL_F32, true, true, false, true, true, false, false>(
        in, second, nullptr, out, n, tid, nthr, &A.flags[size_t(j - 1) * kFlagStride], A.epoch, A.err,
        A.abort_word, A.epoch, A.timeout_ticks, j);
  else
    waited = run_slice<CCL_F32, true, false, false, true, true, false, false>(
        in, in, nullptr, out, n, tid, nthr, &A.flags[size_t(j - 1) * kFlagStride], A.epoch, A.err, A.abort_word,
        A.epoch, A.timeout_ticks, j);
  if (waited < 0) return;  // the whole workgroup leaves together (run_slice's contract)
  wait_vm_stores();
  __syncthreads();
  if (tid == 0) {
    const long long t = wall_clock64();
    if (j == A.hops) A.ticks[1] = t;
    if (j == 0) A.ticks[0] = t;
    if (j < A.hops) slot_flag_store<true>(&A.flags[size_t(j) * kFlagStride], A.epoch, colocated);
  }
}

}  // namespace

int launch_hop_probe(unsigned char* data, unsigned char* second, unsigned long long* flags, unsigned long long* tags,
                     long long* ticks, unsigned int* err_words, unsigned long long* abort_word, unsigned long long epoch,
                     long long timeout_ticks, size_t region, size_t rot, int hops, int bytes, int two_operands,
                     int ll, int nthreads, void* stream, std::string* err) {
  HopArgs A{data, second, flags, tags, ticks, err_words, abort_word, epoch, timeout_ticks, region, rot, hops, bytes,
            two_operands, ll};
  hipLaunchKernelGGL(hop_probe_kernel, dim3(8 * (hops + 1)), dim3(nthreads), 0, reinterpret_cast<hipStream_t>(stream),
                     A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("hop probe launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

}  // namespace ccl
