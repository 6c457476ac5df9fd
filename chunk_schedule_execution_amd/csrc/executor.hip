// Executor kernel for gfx950: one launch runs a whole lowered collective plan.
//
// Every workgroup interprets its own instruction list (rank x workgroup x pipeline
// order, ReSCCL report, section 2.2) with task-level granularity: it runs one
// instruction over all of its slices before the next (ReSCCL report, section 2.1).
// An instruction reads one or two operands (the incoming transfer's staging slot or a
// local buffer, plus an optional local operand to add) and writes one or two
// destinations (a local buffer and/or the next rank's staging slot): the fused
// recv-reduce-copy-send family (MSCCLang report, section 3.1, instruction fusion).
//
// Virtual ranks share the GPU's HBM. A send writes the receiver's slot and
// release-stores the transfer's flag (epoch << 24 | slices done); a recv has one
// thread acquire-poll that flag, then the workgroup reads the slot. Waits are bounded
// by a wall-clock watchdog so that every workgroup always exits.
//
// The data path is HBM-bound streaming (at most one add per 12 bytes moved), so it
// uses 16-byte vector loads/stores, coalesced over the workgroup, with several
// independent loads in flight per thread; no LDS staging and no MFMA.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/ccl.h"
#include "device_abi.h"
#include "executor_device.h"

namespace ccl {
namespace {

// Plain streaming copy: the HBM ceiling a single kernel reaches on this part. Four
// 16-byte vectors per thread in flight, non-temporal loads and stores (the lines are
// not reused), grid-stride; one workgroup per CU streams best here.
__global__ __launch_bounds__(1024) void copy_probe_kernel(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                          int64_t nvec) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    v4u a0 = __builtin_nontemporal_load(src + i), a1 = __builtin_nontemporal_load(src + i + stride);
    v4u a2 = __builtin_nontemporal_load(src + i + 2 * stride), a3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a0, dst + i);
    __builtin_nontemporal_store(a1, dst + i + stride);
    __builtin_nontemporal_store(a2, dst + i + 2 * stride);
    __builtin_nontemporal_store(a3, dst + i + 3 * stride);
  }
  for (; i < nvec; i += stride) dst[i] = src[i];
}

// ---- message-passing litmus test of the transfer-store policy --------------------
//
// Pairs of workgroups exchange fresh data every round with exactly the executor's
// stores, flags and loads: the producer writes the round's words with plain stores
// (the XCD-local transfer stores), waits for them, and sets the flag with a plain store
// when the consumer published the producer's own XCD, else with a full agent-scope
// release (slot_flag_store); the consumer polls the flag with agent-scope loads and
// reads the words with agent-coherent (sc1) loads, as every receive does, compares them
// with the round's values and acknowledges. Every wait is bounded by the watchdog; any
// mismatch or expiry stops all pairs.
struct LitmusArgs {
  unsigned char* data;        // npairs regions of `words` 32-bit words, 256-byte aligned
  unsigned long long* flags;  // per pair, kFlagStride apart: round the producer published
  unsigned long long* acks;   // per pair, kFlagStride apart: round the consumer finished reading
  unsigned long long* tags;   // per workgroup: 1 << 8 | 0x10 | XCD id
  long long* results;         // per pair 8 values (see ccl_litmus_message_passing)
  unsigned long long* stop;
  int npairs, rounds, words, cross;
  long long timeout_ticks;
};

__device__ __forceinline__ uint32_t litmus_value(int pair, int round, int i) {
  uint32_t h = uint32_t(round) * 0x9E3779B1u ^ uint32_t(i) * 0x85EBCA77u ^ uint32_t(pair) * 0xC2B2AE3Du;
  h ^= h >> 15;
  return h * 0x2C1B3C6Du;
}

// Thread 0: spin until the word at p satisfies (tag ? (v >> 8) == 1 : v >= target), the
// watchdog expires or another workgroup stops the test. Returns the word, 0 on give-up.
__device__ unsigned long long litmus_wait(unsigned long long* p, unsigned long long target, bool tag,
                                          const LitmusArgs& A, long long* res) {
  const long long t0 = wall_clock64();
  for (unsigned it = 0;; ++it) {
    const unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tag ? (v >> 8) == 1ull : v >= target) return v;
    if ((it & 15) == 15) {
      if (__hip_atomic_load(A.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return 0;
      if (wall_clock64() - t0 > A.timeout_ticks) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&res[7]), 1ull);
        __hip_atomic_store(A.stop, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__global__ __launch_bounds__(256) void litmus_mp_kernel(LitmusArgs A) {
  __shared__ int s_go, s_bad;
  const int b = blockIdx.x, tid = threadIdx.x, nthr = blockDim.x;
  const unsigned long long my_tag = (1ull << 8) | 0x10ull | xcd_id();
  if (tid == 0) __hip_atomic_store(&A.tags[b], my_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool producer = b < A.npairs;
  const int q = b - A.npairs;
  const int pair = producer ? b : (A.cross ? (q + A.npairs - 1) % A.npairs : q);
  const int peer = producer ? A.npairs + (A.cross ? (pair + 1) % A.npairs : pair) : pair;
  long long* res = A.results + 8 * pair;
  const size_t region = (size_t(A.words) * 4 + 255) / 256 * 256;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(A.data + size_t(pair) * region, A.words * 4);
  unsigned long long* flag = A.flags + size_t(pair) * kFlagStride;
  unsigned long long* ack = A.acks + size_t(pair) * kFlagStride;
  const int nvec = A.words / 4;
  if (tid == 0) {
    res[producer ? 0 : 1] = (long long)(my_tag & 15ull);
    const unsigned long long pt = litmus_wait(&A.tags[peer], 0, true, A, res);
    s_go = pt != 0;
    s_bad = pt == my_tag ? 1 : 0;  // producer: the consumer shares this XCD
  }
  __syncthreads();
  if (!s_go) return;
  const bool colocated = s_bad != 0;
  for (int r = 1; r <= A.rounds; ++r) {
    if (producer) {
      if (r > 1) {
        if (tid == 0) s_go = litmus_wait(ack, (unsigned long long)(r - 1), false, A, res) != 0;
        __syncthreads();
        if (!s_go) return;
      }
      for (int v = tid; v < nvec; v += nthr) {
        const v4u x = {litmus_value(pair, r, 4 * v), litmus_value(pair, r, 4 * v + 1),
                       litmus_value(pair, r, 4 * v + 2), litmus_value(pair, r, 4 * v + 3)};
        st16<kCpolNone>(rsrc, 16 * v, x);
      }
      wait_vm_stores();
      __syncthreads();
      if (tid == 0) {
        slot_flag_store<true>(flag, (unsigned long long)r, colocated);
        if (colocated) res[6] += 1;
      }
    } else {
      if (tid == 0) {
        s_go = litmus_wait(flag, (unsigned long long)r, false, A, res) != 0;
        s_bad = 0;
      }
      __syncthreads();
      if (!s_go) return;
      int bad = 0, first = -1;
      for (int v = tid; v < nvec; v += nthr) {
        const v4u x = ld16<kCpolSc1>(rsrc, 16 * v);
        for (int e = 0; e < 4; ++e)
          if (x[e] != litmus_value(pair, r, 4 * v + e)) {
            if (first < 0) first = 4 * v + e;
            ++bad;
          }
      }
      if (bad) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&res[3]), (unsigned long long)bad);
        if (atomicCAS(reinterpret_cast<unsigned long long*>(&res[4]), 0ull, (unsigned long long)r) == 0ull)
          res[5] = first;
        s_bad = 1;
      }
      __syncthreads();
      if (tid == 0) {
        if (s_bad) __hip_atomic_store(A.stop, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        res[2] = r;
        release_store(ack, (unsigned long long)r);  // every read above completed first
      }
      if (s_bad) return;
    }
  }
}

// Placement probe: each workgroup records the XCD it runs on (XCC_ID) and its hardware
// id word (HW_ID: CU, shader array and engine), then stays for `hold_ticks` of the wall
// clock so that later workgroups spread over other compute units.
__global__ __launch_bounds__(64) void cu_probe_kernel(unsigned* out, long long hold_ticks) {
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = xcd_id();
    out[2 * blockIdx.x + 1] = __builtin_amdgcn_s_getreg((4) | (0 << 6) | ((32 - 1) << 11));
    const long long t0 = wall_clock64();
    while (wall_clock64() - t0 < hold_ticks) __builtin_amdgcn_s_sleep(8);
  }
}

}  // namespace

template <int DT>
static void launch_dt(const ExecArgs& args, bool xl, bool nt, dim3 g, dim3 b, hipStream_t s) {
  if (xl && nt) hipLaunchKernelGGL((executor_kernel<DT, true, true>), g, b, 0, s, args);
  else if (xl) hipLaunchKernelGGL((executor_kernel<DT, true, false>), g, b, 0, s, args);
  else if (nt) hipLaunchKernelGGL((executor_kernel<DT, false, true>), g, b, 0, s, args);
  else hipLaunchKernelGGL((executor_kernel<DT, false, false>), g, b, 0, s, args);
}

int launch_executor(const ExecArgs& args, int dtype, bool xcd_local, bool streaming, int nwg, int nthreads,
                    void* stream, std::string* err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(nwg), b(nthreads);
  switch (dtype) {
    case CCL_F32: launch_dt<CCL_F32>(args, xcd_local, streaming, g, b, s); break;
    case CCL_BF16: launch_dt<CCL_BF16>(args, xcd_local, streaming, g, b, s); break;
    case CCL_I32: launch_dt<CCL_I32>(args, xcd_local, streaming, g, b, s); break;
    default: *err = "dtype"; return CCL_ERR_UNSUPPORTED;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("kernel launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

template <int DT>
static hipError_t min_blocks(int nthreads, int* blocks) {
  int b[4] = {0, 0, 0, 0};
  hipError_t e[4] = {hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[0], executor_kernel<DT, false, false>, nthreads, 0),
                     hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[1], executor_kernel<DT, false, true>, nthreads, 0),
                     hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[2], executor_kernel<DT, true, false>, nthreads, 0),
                     hipOccupancyMaxActiveBlocksPerMultiprocessor(&b[3], executor_kernel<DT, true, true>, nthreads, 0)};
  int m = b[0];
  for (int i = 0; i < 4; ++i) {
    if (e[i] != hipSuccess) return e[i];
    m = b[i] < m ? b[i] : m;
  }
  *blocks = m;
  return hipSuccess;
}

// Every kernel variant of a dtype: the smallest occupancy bounds the plan.
int executor_max_blocks_per_cu(int dtype, int nthreads, int* blocks, std::string* err) {
  hipError_t e = hipSuccess;
  switch (dtype) {
    case CCL_F32: e = min_blocks<CCL_F32>(nthreads, blocks); break;
    case CCL_BF16: e = min_blocks<CCL_BF16>(nthreads, blocks); break;
    case CCL_I32: e = min_blocks<CCL_I32>(nthreads, blocks); break;
    default: *err = "dtype"; return CCL_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) {
    *err = std::string("occupancy query: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

int launch_litmus_mp(unsigned char* data, unsigned long long* flags, unsigned long long* acks,
                     unsigned long long* tags, long long* results, unsigned long long* stop, int npairs, int rounds,
                     int words, int cross, long long timeout_ticks, void* stream, std::string* err) {
  LitmusArgs A{data, flags, acks, tags, results, stop, npairs, rounds, words, cross, timeout_ticks};
  hipLaunchKernelGGL(litmus_mp_kernel, dim3(2 * npairs), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("litmus launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

int launch_cu_probe(unsigned* out, int nblocks, long long hold_ticks, void* stream, std::string* err) {
  hipLaunchKernelGGL(cu_probe_kernel, dim3(nblocks), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), out,
                     hold_ticks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("placement probe launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

int launch_copy_probe(void* dst, const void* src, size_t bytes, int nblocks, int nthreads, void* stream,
                      std::string* err) {
  hipLaunchKernelGGL(copy_probe_kernel, dim3(nblocks), dim3(nthreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<v4u*>(dst), reinterpret_cast<const v4u*>(src), int64_t(bytes / 16));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("copy probe launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

}  // namespace ccl

