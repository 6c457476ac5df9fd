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

namespace ccl {
namespace {

__device__ __forceinline__ int64_t cbound(int64_t j, int64_t N, int64_t C) { return (j * N) / C; }

__device__ __forceinline__ void range_of(int idx, int cnt, int inst, int k, int64_t N, int64_t C, int64_t& lo,
                                         int64_t& len) {
  int64_t a = cbound(idx, N, C), b = cbound(idx + cnt, N, C);
  if (k > 1) {
    int64_t l = b - a;
    int64_t s = a + (inst * l) / k, e = a + ((inst + 1) * l) / k;
    lo = s;
    len = e - s;
  } else {
    lo = a;
    len = b - a;
  }
}

// ---- element arithmetic --------------------------------------------------

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int DT>
struct Arith;

template <>
struct Arith<CCL_F32> {
  static constexpr int esz = 4;
  typedef uint32_t S;
  static __device__ __forceinline__ S add(S a, S b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); }
  static __device__ __forceinline__ uint4 add4(uint4 a, uint4 b) {
    return make_uint4(add(a.x, b.x), add(a.y, b.y), add(a.z, b.z), add(a.w, b.w));
  }
};

template <>
struct Arith<CCL_I32> {
  static constexpr int esz = 4;
  typedef uint32_t S;
  static __device__ __forceinline__ S add(S a, S b) { return a + b; }  // two's-complement wrap
  static __device__ __forceinline__ uint4 add4(uint4 a, uint4 b) {
    return make_uint4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  }
};

template <>
struct Arith<CCL_BF16> {
  static constexpr int esz = 2;
  typedef uint16_t S;
  static __device__ __forceinline__ S add(S a, S b) {
    float s = __uint_as_float(uint32_t(a) << 16) + __uint_as_float(uint32_t(b) << 16);
    return S(f32_to_bf16_bits(s));
  }
  static __device__ __forceinline__ uint32_t add2(uint32_t a, uint32_t b) {
    float lo = __uint_as_float(a << 16) + __uint_as_float(b << 16);
    float hi = __uint_as_float(a & 0xffff0000u) + __uint_as_float(b & 0xffff0000u);
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  static __device__ __forceinline__ uint4 add4(uint4 a, uint4 b) {
    return make_uint4(add2(a.x, b.x), add2(a.y, b.y), add2(a.z, b.z), add2(a.w, b.w));
  }
};

// ---- one slice of one instruction ------------------------------------------

// Indices inside a slice are 32-bit: a slice is at most 2^31 bytes.
template <int DT, bool SRCB, bool DSTA, bool SEND>
__device__ __attribute__((noinline)) void run_slice(const unsigned char* __restrict__ pa,
                                                    const unsigned char* __restrict__ pb,
                                                    unsigned char* __restrict__ pd, unsigned char* __restrict__ pt,
                                                    int n, int tid, int nthr) {
  typedef Arith<DT> Ar;
  typedef typename Ar::S S;
  constexpr int esz = Ar::esz;
  constexpr int V = 16 / esz;
  const uintptr_t ra = uintptr_t(pa) & 15;
  bool same = true;
  if (SRCB) same &= (uintptr_t(pb) & 15) == ra;
  if (DSTA) same &= (uintptr_t(pd) & 15) == ra;
  if (SEND) same &= (uintptr_t(pt) & 15) == ra;
  auto scalar = [&](int e) {
    S v = reinterpret_cast<const S*>(pa)[e];
    if (SRCB) v = Ar::add(v, reinterpret_cast<const S*>(pb)[e]);
    if (DSTA) reinterpret_cast<S*>(pd)[e] = v;
    if (SEND) reinterpret_cast<S*>(pt)[e] = v;
  };
  if (!same) {
    // operands disagree on 16-byte alignment: element-wise, four in flight per thread
    int e = tid;
    for (; e + 3 * nthr < n; e += 4 * nthr) {
      S v0 = reinterpret_cast<const S*>(pa)[e];
      S v1 = reinterpret_cast<const S*>(pa)[e + nthr];
      S v2 = reinterpret_cast<const S*>(pa)[e + 2 * nthr];
      S v3 = reinterpret_cast<const S*>(pa)[e + 3 * nthr];
      if (SRCB) {
        v0 = Ar::add(v0, reinterpret_cast<const S*>(pb)[e]);
        v1 = Ar::add(v1, reinterpret_cast<const S*>(pb)[e + nthr]);
        v2 = Ar::add(v2, reinterpret_cast<const S*>(pb)[e + 2 * nthr]);
        v3 = Ar::add(v3, reinterpret_cast<const S*>(pb)[e + 3 * nthr]);
      }
      if (DSTA) {
        reinterpret_cast<S*>(pd)[e] = v0;
        reinterpret_cast<S*>(pd)[e + nthr] = v1;
        reinterpret_cast<S*>(pd)[e + 2 * nthr] = v2;
        reinterpret_cast<S*>(pd)[e + 3 * nthr] = v3;
      }
      if (SEND) {
        reinterpret_cast<S*>(pt)[e] = v0;
        reinterpret_cast<S*>(pt)[e + nthr] = v1;
        reinterpret_cast<S*>(pt)[e + 2 * nthr] = v2;
        reinterpret_cast<S*>(pt)[e + 3 * nthr] = v3;
      }
    }
    for (; e < n; e += nthr) scalar(e);
    return;
  }
  int head = int((16 - ra) & 15) / esz;
  if (head > n) head = n;
  if (tid < head) scalar(tid);
  const int nvec = (n - head) / V;
  const int off = head * esz;
  const uint4* __restrict__ A4 = reinterpret_cast<const uint4*>(pa + off);
  const uint4* __restrict__ B4 = reinterpret_cast<const uint4*>(SRCB ? pb + off : pa + off);
  uint4* __restrict__ D4 = reinterpret_cast<uint4*>(DSTA ? pd + off : nullptr);
  uint4* __restrict__ T4 = reinterpret_cast<uint4*>(SEND ? pt + off : nullptr);
  int i = tid;
  for (; i + 3 * nthr < nvec; i += 4 * nthr) {
    uint4 a0 = A4[i], a1 = A4[i + nthr], a2 = A4[i + 2 * nthr], a3 = A4[i + 3 * nthr];
    if (SRCB) {
      uint4 b0 = B4[i], b1 = B4[i + nthr], b2 = B4[i + 2 * nthr], b3 = B4[i + 3 * nthr];
      a0 = Ar::add4(a0, b0);
      a1 = Ar::add4(a1, b1);
      a2 = Ar::add4(a2, b2);
      a3 = Ar::add4(a3, b3);
    }
    if (DSTA) {
      D4[i] = a0;
      D4[i + nthr] = a1;
      D4[i + 2 * nthr] = a2;
      D4[i + 3 * nthr] = a3;
    }
    if (SEND) {
      T4[i] = a0;
      T4[i + nthr] = a1;
      T4[i + 2 * nthr] = a2;
      T4[i + 3 * nthr] = a3;
    }
  }
  for (; i < nvec; i += nthr) {
    uint4 a = A4[i];
    if (SRCB) a = Ar::add4(a, B4[i]);
    if (DSTA) D4[i] = a;
    if (SEND) T4[i] = a;
  }
  const int tail0 = head + nvec * V;
  for (int e = tail0 + tid; e < n; e += nthr) scalar(e);
}

template <int DT>
__device__ __forceinline__ void dispatch_slice(uint32_t op, const unsigned char* pa, const unsigned char* pb,
                                               unsigned char* pd, unsigned char* pt, int n, int tid, int nthr) {
  switch (op & (OPB_SRCB | OPB_DSTA | OPB_SEND)) {
    case OPB_DSTA: run_slice<DT, false, true, false>(pa, pb, pd, pt, n, tid, nthr); break;
    case OPB_SEND: run_slice<DT, false, false, true>(pa, pb, pd, pt, n, tid, nthr); break;
    case OPB_DSTA | OPB_SEND: run_slice<DT, false, true, true>(pa, pb, pd, pt, n, tid, nthr); break;
    case OPB_SRCB | OPB_DSTA: run_slice<DT, true, true, false>(pa, pb, pd, pt, n, tid, nthr); break;
    case OPB_SRCB | OPB_SEND: run_slice<DT, true, false, true>(pa, pb, pd, pt, n, tid, nthr); break;
    case OPB_SRCB | OPB_DSTA | OPB_SEND: run_slice<DT, true, true, true>(pa, pb, pd, pt, n, tid, nthr); break;
    default: break;  // an instruction always stores somewhere; the compiler never emits this
  }
}

// ---- flags ------------------------------------------------------------------

__device__ __forceinline__ void release_store(unsigned long long* p, unsigned long long v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void report_timeout(const ExecArgs& A, int instr) {
  if (atomicCAS(&A.err[0], 0u, unsigned(-CCL_ERR_TIMEOUT)) == 0u) {
    A.err[1] = blockIdx.x;
    A.err[2] = unsigned(instr);
    A.err[3] = unsigned(A.epoch);
  }
  __hip_atomic_store(A.abort_word, A.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 only: spin until *p >= target (acquire), the watchdog expires, or the
// launch is aborted by another workgroup's watchdog. Returns false on the latter two.
__device__ bool wait_geq(unsigned long long* p, unsigned long long target, const ExecArgs& A, int instr,
                         unsigned long long& wait_ticks) {
  unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v >= target) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
  }
  const long long t0 = wall_clock64();
  for (unsigned it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= target) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      wait_ticks += (unsigned long long)(wall_clock64() - t0);
      return true;
    }
    if ((it & 15) == 0) {
      if (wall_clock64() - t0 > A.timeout_ticks) {
        report_timeout(A, instr);
        return false;
      }
      if (__hip_atomic_load(A.abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == A.epoch) return false;
    }
  }
}

// ---- the kernel ---------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(1024) void executor_kernel(ExecArgs A) {
  constexpr int esz = Arith<DT>::esz;
  constexpr int V = 16 / esz;
  __shared__ int s_ok;
  const DevWG W = A.wgs[blockIdx.x];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const unsigned long long E = A.epoch << kEpochShift;
  unsigned long long wait_ticks = 0;
  long long t_begin = 0;
  if (A.trace && tid == 0) t_begin = wall_clock64();
  int ran = 0;
  for (int ii = 0; ii < W.n; ++ii) {
    const DevInstr D = A.ins[W.first + ii];
    const int gi = W.first + ii;
    if (D.nwaits > 0) {
      if (tid == 0) {
        int ok = 1;
        for (int w = 0; w < D.nwaits && ok; ++w)
          ok = wait_geq(&A.dflags[A.waits[D.wait_begin + w]], A.epoch, A, gi, wait_ticks) ? 1 : 0;
        s_ok = ok;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    int64_t lo, len;
    range_of(D.pad0, D.cnt, D.instance, A.k, A.count, A.nchunks, lo, len);
    const unsigned char* pa;
    const unsigned char* pb = nullptr;
    unsigned char* pd = nullptr;
    unsigned char* pt = nullptr;
    if (D.op & OPB_RECV) {
      const DevXfer X = A.xf[D.xin];
      int64_t ph = 0;
      if (X.phase_idx >= 0) {
        int64_t plo, plen;
        range_of(X.phase_idx, X.cnt, X.instance, A.k, A.count, A.nchunks, plo, plen);
        ph = plo % V;
      }
      pa = A.staging + X.slot_off + ph * esz;
    } else {
      int64_t l, n;
      range_of(D.a_idx, D.cnt, D.instance, A.k, A.count, A.nchunks, l, n);
      pa = A.base[D.a_buf][W.rank] + l * esz;
    }
    if (D.op & OPB_SRCB) {
      int64_t l, n;
      range_of(D.b_idx, D.cnt, D.instance, A.k, A.count, A.nchunks, l, n);
      pb = A.base[D.b_buf][W.rank] + l * esz;
    }
    if (D.op & OPB_DSTA) {
      int64_t l, n;
      range_of(D.d_idx, D.cnt, D.instance, A.k, A.count, A.nchunks, l, n);
      pd = A.base[D.d_buf][W.rank] + l * esz;
    }
    if (D.op & OPB_SEND) {
      const DevXfer X = A.xf[D.xout];
      int64_t ph = 0;
      if (X.phase_idx >= 0) {
        int64_t plo, plen;
        range_of(X.phase_idx, X.cnt, X.instance, A.k, A.count, A.nchunks, plo, plen);
        ph = plo % V;
      }
      pt = A.staging + X.slot_off + ph * esz;
    }
    const int64_t se = A.slice_elems;
    const int64_t nsl = (len + se - 1) / se;
    for (int64_t s = 0; s < nsl; ++s) {
      if (D.op & OPB_RECV) {
        if (tid == 0) s_ok = wait_geq(&A.xflags[D.xin], E + (unsigned long long)(s + 1), A, gi, wait_ticks) ? 1 : 0;
        __syncthreads();
        if (!s_ok) return;
      }
      const int64_t o = s * se;
      const int64_t n = (len - o < se) ? (len - o) : se;
      const int64_t bo = o * esz;
      dispatch_slice<DT>(D.op, pa + bo, pb ? pb + bo : nullptr, pd ? pd + bo : nullptr, pt ? pt + bo : nullptr,
                         int(n), tid, nthr);
      __syncthreads();
      if ((D.op & OPB_SEND) && tid == 0) release_store(&A.xflags[D.xout], E + (unsigned long long)(s + 1));
    }
    if (D.done_flag >= 0 && tid == 0) release_store(&A.dflags[D.done_flag], A.epoch);
    ++ran;
  }
  if (A.trace && tid == 0) {
    unsigned long long* t = A.trace + 4 * size_t(W.trace_slot);
    t[0] = (unsigned long long)t_begin;
    t[1] = (unsigned long long)wall_clock64();
    t[2] = wait_ticks;
    t[3] = (unsigned long long)ran;
  }
}

// Plain streaming copy: the HBM ceiling a single kernel reaches on this part.
__global__ __launch_bounds__(1024) void copy_probe_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                          int64_t nvec) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    uint4 a0 = src[i], a1 = src[i + stride], a2 = src[i + 2 * stride], a3 = src[i + 3 * stride];
    dst[i] = a0;
    dst[i + stride] = a1;
    dst[i + 2 * stride] = a2;
    dst[i + 3 * stride] = a3;
  }
  for (; i < nvec; i += stride) dst[i] = src[i];
}

}  // namespace

int launch_executor(const ExecArgs& args, int dtype, int nwg, int nthreads, void* stream, std::string* err) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (dtype) {
    case CCL_F32: hipLaunchKernelGGL(executor_kernel<CCL_F32>, dim3(nwg), dim3(nthreads), 0, s, args); break;
    case CCL_BF16: hipLaunchKernelGGL(executor_kernel<CCL_BF16>, dim3(nwg), dim3(nthreads), 0, s, args); break;
    case CCL_I32: hipLaunchKernelGGL(executor_kernel<CCL_I32>, dim3(nwg), dim3(nthreads), 0, s, args); break;
    default: *err = "dtype"; return CCL_ERR_UNSUPPORTED;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("kernel launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

int executor_max_blocks_per_cu(int dtype, int nthreads, int* blocks, std::string* err) {
  hipError_t e = hipSuccess;
  switch (dtype) {
    case CCL_F32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, executor_kernel<CCL_F32>, nthreads, 0); break;
    case CCL_BF16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, executor_kernel<CCL_BF16>, nthreads, 0); break;
    case CCL_I32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, executor_kernel<CCL_I32>, nthreads, 0); break;
    default: *err = "dtype"; return CCL_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) {
    *err = std::string("occupancy query: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

int launch_copy_probe(void* dst, const void* src, size_t bytes, int nblocks, int nthreads, void* stream,
                      std::string* err) {
  hipLaunchKernelGGL(copy_probe_kernel, dim3(nblocks), dim3(nthreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), int64_t(bytes / 16));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *err = std::string("copy probe launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

}  // namespace ccl
