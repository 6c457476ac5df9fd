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
//
// Every access goes through a buffer descriptor whose size is the operand's slice, so
// an address outside the operand is dropped by the hardware instead of touching
// other memory. Staging-slot data (RECV loads, SEND stores) uses the sc1 cache policy:
// agent-coherent, the same policy the compiler gives relaxed agent-scope atomics, so a
// slot's data is visible across XCDs as soon as the store completes and no L2
// writeback or invalidate is needed around the slot flags.

typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, gfx9 data format
constexpr int kCpolNone = 0;
constexpr int kCpolSc1 = 16;  // agent-scope coherent

// Slice pointers and sizes are wave-uniform; readfirstlane puts them in scalar
// registers so the descriptor is scalar (no per-lane waterfall around each access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const unsigned char* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  void* u = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

template <int CP>
__device__ __forceinline__ v4u ld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, int off, v4u v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int ESZ, int CP>
__device__ __forceinline__ uint32_t ld_elem(__amdgpu_buffer_rsrc_t r, int off) {
  if (ESZ == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP);
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
}
template <int ESZ, int CP>
__device__ __forceinline__ void st_elem(__amdgpu_buffer_rsrc_t r, int off, uint32_t v) {
  if (ESZ == 2)
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, CP);
  else
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP);
}

__device__ __forceinline__ uint4 to_u4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ v4u to_v4(uint4 v) {
  v4u r = {v.x, v.y, v.z, v.w};
  return r;
}

// Indices inside a slice are 32-bit: a slice is far below 2^31 bytes.
template <int DT, bool RECV, bool SRCB, bool DSTA, bool SEND>
__device__ __attribute__((noinline)) void run_slice(const unsigned char* pa, const unsigned char* pb, unsigned char* pd,
                                                    unsigned char* pt, int n, int tid, int nthr) {
  typedef Arith<DT> Ar;
  constexpr int esz = Ar::esz;
  constexpr int V = 16 / esz;
  constexpr int CA = RECV ? kCpolSc1 : kCpolNone;  // first operand: slot or local buffer
  constexpr int CT = kCpolSc1;                      // outgoing slot
  const int bytes = n * esz;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(pa, bytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(SRCB ? pb : pa, bytes);
  const __amdgpu_buffer_rsrc_t rD = make_rsrc(DSTA ? pd : pa, DSTA ? bytes : 0);
  const __amdgpu_buffer_rsrc_t rT = make_rsrc(SEND ? pt : pa, SEND ? bytes : 0);
  const uintptr_t ra = uintptr_t(pa) & 15;
  bool same = true;
  if (SRCB) same &= (uintptr_t(pb) & 15) == ra;
  if (DSTA) same &= (uintptr_t(pd) & 15) == ra;
  if (SEND) same &= (uintptr_t(pt) & 15) == ra;
  auto scalar = [&](int e) {
    const int o = e * esz;
    uint32_t v = ld_elem<esz, CA>(rA, o);
    if (SRCB) v = Ar::add(typename Ar::S(v), typename Ar::S(ld_elem<esz, kCpolNone>(rB, o)));
    if (DSTA) st_elem<esz, kCpolNone>(rD, o, v);
    if (SEND) st_elem<esz, CT>(rT, o, v);
  };
  int tail0 = 0;
  if (same) {
    int head = int((16 - ra) & 15) / esz;
    if (head > n) head = n;
    if (tid < head) scalar(tid);
    const int nvec = (n - head) / V;
    const int base = head * esz;
    int i = tid;
    for (; i + 3 * nthr < nvec; i += 4 * nthr) {
      const int o0 = base + 16 * i, o1 = o0 + 16 * nthr, o2 = o1 + 16 * nthr, o3 = o2 + 16 * nthr;
      uint4 a0 = to_u4(ld16<CA>(rA, o0)), a1 = to_u4(ld16<CA>(rA, o1));
      uint4 a2 = to_u4(ld16<CA>(rA, o2)), a3 = to_u4(ld16<CA>(rA, o3));
      if (SRCB) {
        uint4 b0 = to_u4(ld16<kCpolNone>(rB, o0)), b1 = to_u4(ld16<kCpolNone>(rB, o1));
        uint4 b2 = to_u4(ld16<kCpolNone>(rB, o2)), b3 = to_u4(ld16<kCpolNone>(rB, o3));
        a0 = Ar::add4(a0, b0);
        a1 = Ar::add4(a1, b1);
        a2 = Ar::add4(a2, b2);
        a3 = Ar::add4(a3, b3);
      }
      if (DSTA) {
        st16<kCpolNone>(rD, o0, to_v4(a0));
        st16<kCpolNone>(rD, o1, to_v4(a1));
        st16<kCpolNone>(rD, o2, to_v4(a2));
        st16<kCpolNone>(rD, o3, to_v4(a3));
      }
      if (SEND) {
        st16<CT>(rT, o0, to_v4(a0));
        st16<CT>(rT, o1, to_v4(a1));
        st16<CT>(rT, o2, to_v4(a2));
        st16<CT>(rT, o3, to_v4(a3));
      }
    }
    for (; i < nvec; i += nthr) {
      const int o = base + 16 * i;
      uint4 a = to_u4(ld16<CA>(rA, o));
      if (SRCB) a = Ar::add4(a, to_u4(ld16<kCpolNone>(rB, o)));
      if (DSTA) st16<kCpolNone>(rD, o, to_v4(a));
      if (SEND) st16<CT>(rT, o, to_v4(a));
    }
    tail0 = head + nvec * V;
  }
  // unaligned operands, or the tail: element by element
  for (int e = tail0 + tid; e < n; e += nthr) scalar(e);
}

template <int DT>
__device__ __forceinline__ void dispatch_slice(uint32_t op, const unsigned char* pa, const unsigned char* pb,
                                               unsigned char* pd, unsigned char* pt, int n, int tid, int nthr) {
#define CCL_CASE(R, B, D, T)                                                                                     \
  case ((R) ? OPB_RECV : 0u) | ((B) ? OPB_SRCB : 0u) | ((D) ? OPB_DSTA : 0u) | ((T) ? OPB_SEND : 0u):            \
    run_slice<DT, R, B, D, T>(pa, pb, pd, pt, n, tid, nthr);                                                    \
    break;
  switch (op & 15u) {
    CCL_CASE(false, false, true, false)
    CCL_CASE(false, false, false, true)
    CCL_CASE(false, false, true, true)
    CCL_CASE(false, true, true, false)
    CCL_CASE(false, true, false, true)
    CCL_CASE(false, true, true, true)
    CCL_CASE(true, false, true, false)
    CCL_CASE(true, false, false, true)
    CCL_CASE(true, false, true, true)
    CCL_CASE(true, true, true, false)
    CCL_CASE(true, true, false, true)
    CCL_CASE(true, true, true, true)
    default: break;  // an instruction always stores somewhere; the compiler never emits this
  }
#undef CCL_CASE
}

// ---- flags ------------------------------------------------------------------

// Completion flags guard local-buffer data written with ordinary (L2-cached)
// stores: a full agent-scope release / acquire.
__device__ __forceinline__ void release_store(unsigned long long* p, unsigned long long v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slot flags guard sc1 data whose stores every wave has already waited for.
__device__ __forceinline__ void slot_flag_store(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_vm_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ void report_timeout(const ExecArgs& A, int instr) {
  if (atomicCAS(&A.err[0], 0u, unsigned(-CCL_ERR_TIMEOUT)) == 0u) {
    A.err[1] = blockIdx.x;
    A.err[2] = unsigned(instr);
    A.err[3] = unsigned(A.epoch);
  }
  __hip_atomic_store(A.abort_word, A.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 only: spin until *p >= target, the watchdog expires, or the launch is
// aborted by another workgroup's watchdog. Returns false on the latter two. With
// ACQ the success path ends in an agent-scope acquire fence.
template <bool ACQ>
__device__ bool wait_geq(unsigned long long* p, unsigned long long target, const ExecArgs& A, int instr,
                         unsigned long long& wait_ticks) {
  unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v >= target) {
    if (ACQ) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
  }
  const long long t0 = wall_clock64();
  for (unsigned it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= target) {
      if (ACQ) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
  __shared__ int s_ok;
  const DevWG W = A.wgs[blockIdx.x];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const unsigned long long E = A.epoch << kEpochShift;
  unsigned long long wait_ticks = 0;
  long long t_begin = 0;
  if (A.trace && tid == 0) t_begin = wall_clock64();
  int ran = 0;
  for (int ii = 0; ii < W.n; ++ii) {
    const int gi = W.first + ii;
    const DevInstr D = A.ins[gi];
    const DevGeo G = A.geo[gi];
    if (D.nwaits > 0) {
      if (tid == 0) {
        int ok = 1;
        for (int w = 0; w < D.nwaits && ok; ++w)
          ok = wait_geq<true>(&A.dflags[A.waits[D.wait_begin + w]], A.epoch, A, gi, wait_ticks) ? 1 : 0;
        s_ok = ok;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    const unsigned char* pa =
        (D.op & OPB_RECV) ? A.staging + G.a_off : A.base[D.a_buf][W.rank] + G.a_off;
    const unsigned char* pb = (D.op & OPB_SRCB) ? A.base[D.b_buf][W.rank] + G.b_off : nullptr;
    unsigned char* pd = (D.op & OPB_DSTA) ? A.base[D.d_buf][W.rank] + G.d_off : nullptr;
    unsigned char* pt = (D.op & OPB_SEND) ? A.staging + G.t_off : nullptr;
    const int64_t se = A.slice_elems;
    for (int64_t s = 0; s < G.nsl; ++s) {
      if (D.op & OPB_RECV) {
        if (tid == 0)
          s_ok = wait_geq<false>(&A.xflags[D.xin], E + (unsigned long long)(s + 1), A, gi, wait_ticks) ? 1 : 0;
        __syncthreads();
        if (!s_ok) return;
      }
      const int64_t o = s * se;
      const int n = int((G.len - o < se) ? (G.len - o) : se);
      const int64_t bo = o * esz;
      dispatch_slice<DT>(D.op, pa + bo, pb ? pb + bo : nullptr, pd ? pd + bo : nullptr, pt ? pt + bo : nullptr, n,
                         tid, nthr);
      if (D.op & OPB_SEND) wait_vm_stores();
      __syncthreads();
      if ((D.op & OPB_SEND) && tid == 0) slot_flag_store(&A.xflags[D.xout], E + (unsigned long long)(s + 1));
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
