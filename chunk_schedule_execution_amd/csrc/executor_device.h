// Device code of the executor: element arithmetic, slice and low-latency transfer
// loops, flag waits and stores, the per-instruction step and the interpreting kernel.
// Compiled into the library by executor.hip, and handed as source text to the
// runtime compiler for the plan-specialized kernels, which reuse every piece of it.
// The includer provides <hip/hip_runtime.h>, ccl.h and device_abi.h first.
#pragma once

namespace ccl {
namespace {

// ---- element arithmetic --------------------------------------------------

// fp32 -> bf16, round to nearest, ties to even, in one instruction (v_cvt_pk_bf16_f32,
// two values at a time); a NaN becomes the quiet NaN 0x7fc0 with its sign. Over all 2^32
// fp32 inputs the instruction gives the same bits as the rounding written out,
// (u + 0x7fff + lsb) >> 16, on every non-NaN input; NaNs keep part of their payload
// there, hence the fix-up. Against the written-out rounding it took a bf16 8-rank ring
// at 3 MiB from 38.3 to 35.4 us and at 32 MiB from 189 to 180 us.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  const f32x2 v = {lo, hi};
  uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  if (__builtin_isnan(lo)) r = (r & 0xffff0000u) | ((__float_as_uint(lo) >> 16) & 0x8000u) | 0x7fc0u;
  if (__builtin_isnan(hi)) r = (r & 0x0000ffffu) | (__float_as_uint(hi) & 0x80000000u) | 0x7fc00000u;
  return r;
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
    return S(f32x2_to_bf16x2_bits(s, 0.0f) & 0xffffu);
  }
  static __device__ __forceinline__ uint32_t add2(uint32_t a, uint32_t b) {
    float lo = __uint_as_float(a << 16) + __uint_as_float(b << 16);
    float hi = __uint_as_float(a & 0xffff0000u) + __uint_as_float(b & 0xffff0000u);
    return f32x2_to_bf16x2_bits(lo, hi);
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
constexpr int kCpolNt = 2;    // non-temporal: streamed lines are not kept

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

// Thread 0 only: spin until *p >= target, the watchdog expires, or the launch is
// aborted; returns the ticks spent, or -1 on the latter two.
__device__ __forceinline__ long long wait_slot_flag(unsigned long long* p, unsigned long long target,
                                                    unsigned int* err, unsigned long long* abort_word,
                                                    unsigned long long epoch, long long timeout_ticks, int instr);

// Inlined into the kernel: a call would reload its target and arguments through the
// scalar cache on every slice. Indices inside a slice are 32-bit: a slice is far below
// 2^31 bytes. With RECV, the slice first waits for the incoming slot flag (*wflag >=
// wtarget).
// Returns the ticks waited, or -1 if the wait gave up (the whole workgroup returns
// -1 together).
template <int DT, bool RECV, bool SRCB, bool DSTA, bool SEND, bool XL, bool NT, bool NF>
__device__ __forceinline__ long long run_slice(const unsigned char* pa, const unsigned char* pb,
                                                         unsigned char* pd, unsigned char* pt, int n, int tid,
                                                         int nthr, unsigned long long* wflag,
                                                         unsigned long long wtarget, unsigned int* err,
                                                         unsigned long long* abort_word, unsigned long long epoch,
                                                         long long timeout_ticks, int instr) {
  __shared__ long long s_waited;
  typedef Arith<DT> Ar;
  constexpr int esz = Ar::esz;
  constexpr int V = 16 / esz;
  constexpr int CL = NT ? kCpolNt : kCpolNone;      // local-buffer loads and stores
  constexpr int CA = RECV ? kCpolSc1 : CL;          // first operand: slot or local buffer
  // outgoing data: plain (XCD-local layout) or coherent; a flagless send (NF: its receive
  // is skipped, nothing reads the data before the launch ends) streams like local stores
  constexpr int CT = NF ? CL : XL ? kCpolNone : kCpolSc1;
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
    if (SRCB) v = Ar::add(typename Ar::S(v), typename Ar::S(ld_elem<esz, CL>(rB, o)));
    if (DSTA) st_elem<esz, CL>(rD, o, v);
    if (SEND) st_elem<esz, CT>(rT, o, v);
  };
  int head = 0, nvec = 0, base = 0;
  if (same) {
    head = int((16 - ra) & 15) / esz;
    if (head > n) head = n;
    nvec = (n - head) / V;
    base = head * esz;
  }
  // Vectors per thread per pass: all issued before any is consumed. bf16 takes two,
  // except in the streaming variant (long transfers), where two kept half the loads in
  // flight and streamed 8-12 % slower at 64-256 MiB per rank. At latency-bound sizes four
  // cost 10-17 % when bf16 rounding was emulated; with the hardware conversion they still
  // cost 1 us at 1 MiB (8-rank ring 21.3 -> 22.4 us, 16-rank hierarchical 35.9 -> 37.4)
  // and gained only at 3 MiB (35.6 -> 33.9).
  // Streaming copies and forwards of 32-bit data (one operand) take eight: a 24-rank
  // ring AllGather at 128 MiB went from 68 to 77 % of HBM peak, while eight for two
  // operands ran out of registers (ReduceScatter 69 -> 31 %).
  constexpr int U = (NT && !SRCB && DT != CCL_BF16) ? 8 : (DT == CCL_BF16 && !NT) ? 2 : 4;
  const uint4 zero = {0, 0, 0, 0};
  // First pass of the second operand, loaded before the wait only in the streaming
  // variant (large transfers): a wave's loads complete in order, so the polling wave's
  // flag loads queue behind such early loads, and at latency-bound sizes the steps
  // measured slower with it than without.
  uint4 pf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) pf[u] = zero;
  constexpr bool kPrefetch = SRCB && RECV && NT;
  if (kPrefetch && same) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (tid + u * nthr < nvec) pf[u] = to_u4(ld16<CL>(rB, base + 16 * (tid + u * nthr)));
  }
  long long waited = 0;
  if (RECV) {
    if (tid == 0) s_waited = wait_slot_flag(wflag, wtarget, err, abort_word, epoch, timeout_ticks, instr);
    __syncthreads();
    waited = s_waited;
    if (waited < 0) return -1;
  }
  if constexpr (!DSTA && !SEND) return waited;  // a receive whose data the sender already placed
  int tail0 = 0;
  if (same) {
    if (tid < head) scalar(tid);
    for (int i = tid; i < nvec; i += U * nthr) {
      uint4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[u] = zero;
        if (i + u * nthr < nvec) a[u] = to_u4(ld16<CA>(rA, base + 16 * (i + u * nthr)));
      }
      if (SRCB) {
        uint4 bb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          bb[u] = zero;
          if (kPrefetch && i == tid)
            bb[u] = pf[u];
          else if (i + u * nthr < nvec)
            bb[u] = to_u4(ld16<CL>(rB, base + 16 * (i + u * nthr)));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = Ar::add4(a[u], bb[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i + u * nthr >= nvec) continue;
        const int o = base + 16 * (i + u * nthr);
        if (DSTA) st16<CL>(rD, o, to_v4(a[u]));
        if (SEND) st16<CT>(rT, o, to_v4(a[u]));
      }
    }
    tail0 = head + nvec * V;
  }
  // Operands at different 16-byte phases (shards whose size is no multiple of 16 bytes:
  // the last hop of a ReduceScatter chain reads at the shard's offset and writes the
  // output at 0), or the tail: element by element. Reducing slices of the streaming
  // variant (long transfers, where such pieces are long) load eight elements per thread
  // before using any, so a piece takes a few dependent passes instead of one per
  // workgroup-width of elements: a 24-rank ReduceScatter at 128 MiB with shards off the
  // 16-byte grid ran 4 % faster. Everything else keeps the short loop: the unrolled one
  // cost latency-bound rings 2 % (more scalar registers spilled on every path) and a
  // 24-rank AllGather 1 % (its longer straight-line code).
  if constexpr (!NT || !SRCB) {
    for (int e = tail0 + tid; e < n; e += nthr) scalar(e);
    return waited;
  }
  constexpr int UE = 8;
  for (int e0 = tail0 + tid; e0 < n; e0 += UE * nthr) {
    uint32_t v[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) v[u] = e0 + u * nthr < n ? ld_elem<esz, CA>(rA, (e0 + u * nthr) * esz) : 0u;
    uint32_t w[UE];
#pragma unroll
    for (int u = 0; u < UE; ++u) w[u] = e0 + u * nthr < n ? ld_elem<esz, CL>(rB, (e0 + u * nthr) * esz) : 0u;
#pragma unroll
    for (int u = 0; u < UE; ++u) v[u] = Ar::add(typename Ar::S(v[u]), typename Ar::S(w[u]));
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int e = e0 + u * nthr;
      if (e >= n) continue;
      if (DSTA) st_elem<esz, CL>(rD, e * esz, v[u]);
      if (SEND) st_elem<esz, CT>(rT, e * esz, v[u]);
    }
  }
  return waited;
}

// bf16 widening adds need more registers. In the interpreting kernel, which holds every
// operation's slice code, bf16 slices stay an out-of-line call so the register
// allocator sees one variant at a time (no spills). Generated kernels inline them like
// fp32 / int32: each step there is one fixed operation, and a call site makes the
// caller keep its live values in callee-saved registers (bf16 hierarchical AllReduce:
// 103 -> 89 VGPRs and no scratch; 1 MiB 40.6 -> 36.8 us; bf16 8-rank ring at 3 MiB
// 42.9 -> 38.4 us, at 32 MiB 200 -> 189 us).
template <int DT, bool RECV, bool SRCB, bool DSTA, bool SEND, bool XL, bool NT, bool NF>
__device__ __attribute__((noinline)) long long run_slice_call(const unsigned char* pa, const unsigned char* pb,
                                                              unsigned char* pd, unsigned char* pt, int n, int tid,
                                                              int nthr, unsigned long long* wflag,
                                                              unsigned long long wtarget, unsigned int* err,
                                                              unsigned long long* abort_word, unsigned long long epoch,
                                                              long long timeout_ticks, int instr) {
  return run_slice<DT, RECV, SRCB, DSTA, SEND, XL, NT, NF>(pa, pb, pd, pt, n, tid, nthr, wflag, wtarget, err,
                                                           abort_word, epoch, timeout_ticks, instr);
}

// nf: a flagless send (OPB_NOFLAG); it changes the store policy only in the streaming
// variant of generated kernels (SPEC: the operation word is a compile-time constant, so
// one form is compiled; SPEC also inlines bf16 slices). The interpreting kernel keeps a single form: a second set of
// slice loops made its streaming variant twice as slow (register pressure).
template <int DT, bool XL, bool NT, bool SPEC>
__device__ __forceinline__ long long dispatch_slice(uint32_t op, bool nf, const unsigned char* pa,
                                                    const unsigned char* pb, unsigned char* pd, unsigned char* pt,
                                                    int n, int tid, int nthr, unsigned long long* wflag,
                                                    unsigned long long wtarget, const ExecArgs& A, int instr) {
#define CCL_CALL(R, B, D, T, F)                                                                                  \
  ((DT == CCL_BF16 && !SPEC) ? run_slice_call<DT, R, B, D, T, XL, NT, F>(pa, pb, pd, pt, n, tid, nthr, wflag, wtarget, \
                                                              A.err, A.abort_word, A.epoch, A.timeout_ticks,     \
                                                              instr)                                             \
                    : run_slice<DT, R, B, D, T, XL, NT, F>(pa, pb, pd, pt, n, tid, nthr, wflag, wtarget, A.err,   \
                                                           A.abort_word, A.epoch, A.timeout_ticks, instr))
#define CCL_CASE(R, B, D, T)                                                                                     \
  case ((R) ? OPB_RECV : 0u) | ((B) ? OPB_SRCB : 0u) | ((D) ? OPB_DSTA : 0u) | ((T) ? OPB_SEND : 0u):            \
    if constexpr (SPEC && NT && (T)) {                                                                           \
      if (nf) return CCL_CALL(R, B, D, T, true);                                                                 \
    }                                                                                                            \
    return CCL_CALL(R, B, D, T, false);
  switch (op & 15u) {
    CCL_CASE(false, false, true, false)
    CCL_CASE(false, false, false, true)
    CCL_CASE(false, false, true, true)
    CCL_CASE(false, true, true, false)
    CCL_CASE(false, true, false, true)
    CCL_CASE(false, true, true, true)
    CCL_CASE(true, false, false, false)
    CCL_CASE(true, false, true, false)
    CCL_CASE(true, false, false, true)
    CCL_CASE(true, false, true, true)
    CCL_CASE(true, true, true, false)
    CCL_CASE(true, true, false, true)
    CCL_CASE(true, true, true, true)
    default: return 0;  // every other instruction stores somewhere; the compiler never emits these
  }
#undef CCL_CASE
#undef CCL_CALL
}

// ---- low-latency protocol ------------------------------------------------------
//
// A slot holds 8-byte units {4 data bytes, 4-byte flag}; the flag of every unit of
// this launch is A.ll_flag. A sender writes units with sc1 stores and needs no
// barrier or separate flag; a receiver thread polls exactly the units it consumes.
// Each thread handles quads (4 units = 16 data bytes) when every local operand is
// 16-byte aligned, else single units. Returns true if this thread gave up
// (watchdog or another workgroup's abort); the caller makes the workgroup leave
// together at its next barrier.

typedef unsigned v2u __attribute__((ext_vector_type(2)));

struct WaitCtx {
  unsigned int* err;
  unsigned long long* abort_word;
  unsigned long long epoch;
  long long timeout_ticks;
  int instr;
};

__device__ __noinline__ bool ll_give_up_slow(unsigned int* err, unsigned long long* abort_word,
                                             unsigned long long epoch, long long timeout_ticks, int instr,
                                             long long t0) {
  if (timeout_ticks < 0 || wall_clock64() - t0 > timeout_ticks) {
    if (atomicCAS(&err[0], 0u, unsigned(-CCL_ERR_TIMEOUT)) == 0u) {
      err[1] = blockIdx.x;
      err[2] = unsigned(instr);
      err[3] = unsigned(epoch);
    }
    __hip_atomic_store(abort_word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  return __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
}
__device__ __forceinline__ bool ll_give_up(const WaitCtx& w, long long t0) {
  return ll_give_up_slow(w.err, w.abort_word, w.epoch, w.timeout_ticks, w.instr, t0);
}

// 4 units (32 bytes) at byte offset off; returns their data words.
__device__ __forceinline__ bool ll_load_quad(__amdgpu_buffer_rsrc_t r, int off, uint32_t flag, const WaitCtx& w,
                                             v4u& out) {
  v4u x = ld16<kCpolSc1>(r, off), y = ld16<kCpolSc1>(r, off + 16);
  if (x.y != flag || x.w != flag || y.y != flag || y.w != flag) {
    const long long t0 = wall_clock64();
    for (unsigned it = 1;; ++it) {
      __builtin_amdgcn_s_sleep(1);
      x = ld16<kCpolSc1>(r, off);
      y = ld16<kCpolSc1>(r, off + 16);
      if (x.y == flag && x.w == flag && y.y == flag && y.w == flag) break;
      if ((it & 63) == 0 && ll_give_up(w, t0)) return false;
    }
  }
  out.x = x.x;
  out.y = x.z;
  out.z = y.x;
  out.w = y.z;
  return true;
}

__device__ __forceinline__ bool ll_load_unit(__amdgpu_buffer_rsrc_t r, int off, uint32_t flag, const WaitCtx& w,
                                             uint32_t& out) {
  v2u x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolSc1);
  if (x.y != flag) {
    const long long t0 = wall_clock64();
    for (unsigned it = 1;; ++it) {
      __builtin_amdgcn_s_sleep(1);
      x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolSc1);
      if (x.y == flag) break;
      if ((it & 63) == 0 && ll_give_up(w, t0)) return false;
    }
  }
  out = x.x;
  return true;
}

template <int CP>
__device__ __forceinline__ void ll_store_quad(__amdgpu_buffer_rsrc_t r, int off, v4u v, uint32_t flag) {
  v4u a = {v.x, flag, v.y, flag}, b = {v.z, flag, v.w, flag};
  st16<CP>(r, off, a);
  st16<CP>(r, off + 16, b);
}

// One data word (4 bytes of the transfer) of a local operand starting at byte `o`:
// whole for 4-byte types, assembled from two bf16 elements otherwise (the second only
// if it exists).
template <int ESZ>
__device__ __forceinline__ uint32_t ld_word(__amdgpu_buffer_rsrc_t r, int o, bool second) {
  if (ESZ == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, kCpolNone);
  uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, kCpolNone);
  uint32_t hi = second ? uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, o + 2, 0, kCpolNone)) : 0u;
  return lo | (hi << 16);
}
template <int ESZ>
__device__ __forceinline__ void st_word(__amdgpu_buffer_rsrc_t r, int o, uint32_t v, bool second) {
  if (ESZ == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, o, 0, kCpolNone);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v & 0xffffu), r, o, 0, kCpolNone);
    if (second) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v >> 16), r, o + 2, 0, kCpolNone);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t add_word(uint32_t a, uint32_t b) {
  if (DT == CCL_BF16) return Arith<CCL_BF16>::add2(a, b);
  return Arith<DT>::add(a, b);
}

__device__ __forceinline__ unsigned long long use_here(unsigned long long v);

// Whether outgoing LL units may be plain stores: only in the XCD-local layout, and only
// when the receiver's tag for this launch names this workgroup's XCD (here_tag). The
// caller loads the tag before the step's data loads; compared at the first unit store,
// it has returned with them (a wave's loads return in order), so the decision adds no
// wait. Otherwise the units are agent-coherent stores, which need no release after them.
template <bool XL>
__device__ __forceinline__ bool ll_plain_units(unsigned long long peer_tag, unsigned long long here_tag) {
  return XL && __builtin_amdgcn_readfirstlane(uint32_t(use_here(peer_tag) == here_tag)) != 0u;
}

// The wait context travels as separate scalars: a struct argument would go through
// the stack. peer_tag / here_tag: see ll_plain_units (both 0: plain units in the
// XCD-local layout, the caller makes them visible).
template <int DT, bool RECV, bool SRCB, bool DSTA, bool SEND, bool XL>
__device__ __forceinline__ bool run_ll(const unsigned char* pa, const unsigned char* pb, unsigned char* pd,
                                                 unsigned char* pt, int n, int tid, int nthr, uint32_t flag,
                                                 unsigned int* err, unsigned long long* abort_word,
                                                 unsigned long long epoch, long long timeout_ticks, int instr,
                                                 unsigned long long peer_tag = 0, unsigned long long here_tag = 0) {
  const WaitCtx w{err, abort_word, epoch, timeout_ticks, instr};
  typedef Arith<DT> Ar;
  constexpr int esz = Ar::esz;
  const int bytes = n * esz;
  const int nunits = (bytes + 3) / 4;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(pa, RECV ? nunits * 8 : bytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(SRCB ? pb : pa, SRCB ? bytes : 0);
  const __amdgpu_buffer_rsrc_t rD = make_rsrc(DSTA ? pd : pa, DSTA ? bytes : 0);
  const __amdgpu_buffer_rsrc_t rT = make_rsrc(SEND ? pt : pa, SEND ? nunits * 8 : 0);
  bool aligned = true;
  if (!RECV) aligned &= (uintptr_t(pa) & 15) == 0;
  if (SRCB) aligned &= (uintptr_t(pb) & 15) == 0;
  if (DSTA) aligned &= (uintptr_t(pd) & 15) == 0;
  const int nquads = aligned ? bytes / 16 : 0;
  for (int q = tid; q < nquads; q += 2 * nthr) {
    const int q1 = q + nthr;
    const bool has1 = q1 < nquads;
    v4u v0, v1 = {0, 0, 0, 0}, b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
    if (SRCB) {  // the local operand is in flight while the units are polled
      b0 = ld16<kCpolNone>(rB, 16 * q);
      if (has1) b1 = ld16<kCpolNone>(rB, 16 * q1);
    }
    if (RECV) {
      if (!ll_load_quad(rA, 32 * q, flag, w, v0)) return true;
      if (has1 && !ll_load_quad(rA, 32 * q1, flag, w, v1)) return true;
    } else {
      v0 = ld16<kCpolNone>(rA, 16 * q);
      if (has1) v1 = ld16<kCpolNone>(rA, 16 * q1);
    }
    if (SRCB) {
      v0 = to_v4(Ar::add4(to_u4(v0), to_u4(b0)));
      v1 = to_v4(Ar::add4(to_u4(v1), to_u4(b1)));
    }
    if (DSTA) {
      st16<kCpolNone>(rD, 16 * q, v0);
      if (has1) st16<kCpolNone>(rD, 16 * q1, v1);
    }
    if (SEND) {
      if (ll_plain_units<XL>(peer_tag, here_tag)) {
        ll_store_quad<kCpolNone>(rT, 32 * q, v0, flag);
        if (has1) ll_store_quad<kCpolNone>(rT, 32 * q1, v1, flag);
      } else {
        ll_store_quad<kCpolSc1>(rT, 32 * q, v0, flag);
        if (has1) ll_store_quad<kCpolSc1>(rT, 32 * q1, v1, flag);
      }
    }
  }
  for (int u = 4 * nquads + tid; u < nunits; u += nthr) {
    const int o = 4 * u;
    const bool second = (esz == 2) && (o + 2 < bytes);
    uint32_t v, b = 0;
    if (SRCB) b = ld_word<esz>(rB, o, second);
    if (RECV) {
      if (!ll_load_unit(rA, 8 * u, flag, w, v)) return true;
    } else {
      v = ld_word<esz>(rA, o, second);
    }
    if (SRCB) v = add_word<DT>(v, b);
    if (DSTA) st_word<esz>(rD, o, v, second);
    if (SEND) {
      v2u unit = {v, flag};
      if (ll_plain_units<XL>(peer_tag, here_tag))
        __builtin_amdgcn_raw_buffer_store_b64(unit, rT, 8 * u, 0, kCpolNone);
      else
        __builtin_amdgcn_raw_buffer_store_b64(unit, rT, 8 * u, 0, kCpolSc1);
    }
  }
  return false;
}

template <int DT, bool RECV, bool SRCB, bool DSTA, bool SEND, bool XL>
__device__ __attribute__((noinline)) bool run_ll_call(const unsigned char* pa, const unsigned char* pb,
                                                      unsigned char* pd, unsigned char* pt, int n, int tid, int nthr,
                                                      uint32_t flag, unsigned int* err, unsigned long long* abort_word,
                                                      unsigned long long epoch, long long timeout_ticks, int instr,
                                                      unsigned long long peer_tag, unsigned long long here_tag) {
  return run_ll<DT, RECV, SRCB, DSTA, SEND, XL>(pa, pb, pd, pt, n, tid, nthr, flag, err, abort_word, epoch,
                                                timeout_ticks, instr, peer_tag, here_tag);
}

template <int DT, bool XL>
__device__ __forceinline__ bool dispatch_ll(uint32_t op, const unsigned char* pa, const unsigned char* pb,
                                            unsigned char* pd, unsigned char* pt, int n, int tid, int nthr,
                                            uint32_t flag, const WaitCtx& w, unsigned long long peer_tag,
                                            unsigned long long here_tag) {
#define CCL_CASE(R, B, D, T)                                                                                      \
  case ((R) ? OPB_RECV : 0u) | ((B) ? OPB_SRCB : 0u) | ((D) ? OPB_DSTA : 0u) | ((T) ? OPB_SEND : 0u):             \
    return (DT == CCL_BF16) ? run_ll_call<DT, R, B, D, T, XL>(pa, pb, pd, pt, n, tid, nthr, flag, w.err,         \
                                                              w.abort_word, w.epoch, w.timeout_ticks, w.instr,   \
                                                              peer_tag, here_tag)                                \
                            : run_ll<DT, R, B, D, T, XL>(pa, pb, pd, pt, n, tid, nthr, flag, w.err, w.abort_word, \
                                                         w.epoch, w.timeout_ticks, w.instr, peer_tag, here_tag);
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
    default: return false;
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

// Transfer flags. Coherent layouts write the data with agent-coherent stores, so a
// relaxed agent-scope flag store after every wave's stores are acknowledged suffices.
// XCD-local layouts write the data with plain stores, which stay in the writer's XCD
// L2: when the receiving workgroup runs on the same XCD (its tag for this launch says
// so) that L2 is the point both sides share and the flag is a plain store too;
// otherwise the flag store is a full agent-scope release (L2 writeback first).
// Receivers read flags and data with agent-coherent loads either way.
template <bool XL>
__device__ __forceinline__ void slot_flag_store(unsigned long long* p, unsigned long long v, bool colocated) {
  if (XL && colocated) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    if (XL) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Keeps the compiler from moving the first use of a loaded value above this point (the
// wait for the load lands here, after the instruction's own memory traffic).
__device__ __forceinline__ unsigned long long use_here(unsigned long long v) {
  uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
  asm volatile("" : "+v"(lo), "+v"(hi));
  return (uint64_t(hi) << 32) | lo;
}

// XCD of the executing workgroup (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ unsigned xcd_id() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)); }

__device__ __forceinline__ void wait_vm_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

__device__ void report_timeout(const ExecArgs& A, int instr) {
  if (atomicCAS(&A.err[0], 0u, unsigned(-CCL_ERR_TIMEOUT)) == 0u) {
    A.err[1] = blockIdx.x;
    A.err[2] = unsigned(instr);
    A.err[3] = unsigned(A.epoch);
  }
  __hip_atomic_store(A.abort_word, A.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ long long wait_slot_flag(unsigned long long* p, unsigned long long target,
                                                    unsigned int* err, unsigned long long* abort_word,
                                                    unsigned long long epoch, long long timeout_ticks, int instr) {
  unsigned long long v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v >= target) return 0;
  const long long t0 = wall_clock64();
  for (unsigned it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= target) return wall_clock64() - t0;
    if ((it & 15) == 0) {
      if (wall_clock64() - t0 > timeout_ticks) {
        ll_give_up_slow(err, abort_word, epoch, -1, instr, t0);  // records the timeout and aborts
        return -1;
      }
      if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) return -1;
    }
  }
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

// Records held in LDS at a time: each workgroup copies its instruction records in
// blocks of this many (80 bytes each) and reads them from LDS, so the per-instruction
// path touches no global table.
constexpr int kLdsRecs = 128;

__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Per-workgroup state of one launch, shared by the interpreting kernel below and the
// plan-specialized kernels generated at plan creation.
struct WgState {
  unsigned char *buf0, *buf1, *buf2;  // this rank's buffers, kept in scalar registers
  unsigned char* staging;
  unsigned long long my_tag, E, wait_ticks;
  unsigned long long* itrace;
  long long t_begin;
  int* s_abort;
  int tid, nthr;
};

template <bool XL>
// nthr: the workgroup size. Straight-line generated kernels pass it as a constant:
// blockDim.x is a load from the implicit kernel arguments that every workgroup would wait
// for before its first instruction. Loop-form and interpreting kernels pass blockDim.x
// (with a constant or argument value the compiler scheduled some of their loops worse).
__device__ __forceinline__ void wg_begin(const ExecArgs& A, const DevWG& W, WgState& S, int* s_abort, int nthr) {
  S.tid = threadIdx.x;
  S.nthr = nthr;
  // This workgroup's XCD for this launch, published for the workgroups that send to it.
  S.my_tag = (A.epoch << 8) | 0x10ull | xcd_id();
  if (XL && A.xcd_tags && S.tid == 0)
    __hip_atomic_store(&A.xcd_tags[blockIdx.x], S.my_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  S.E = A.epoch << kEpochShift;
  S.buf0 = A.base[0][W.rank];
  S.buf1 = A.base[1][W.rank];
  S.buf2 = A.base[2][W.rank];
  S.staging = A.staging;
  S.wait_ticks = 0;
  S.t_begin = 0;
  if (A.trace && S.tid == 0) S.t_begin = wall_clock64();
  S.itrace = A.trace ? A.trace + 4 * size_t(gridDim.x) : nullptr;
  S.s_abort = s_abort;
  if (S.tid == 0) *s_abort = 0;
}

__device__ __forceinline__ void wg_end(const ExecArgs& A, const DevWG& W, const WgState& S, int ran) {
  if (A.trace && S.tid == 0) {
    unsigned long long* t = A.trace + 4 * size_t(W.trace_slot);
    t[0] = (unsigned long long)S.t_begin;
    t[1] = (unsigned long long)wall_clock64();
    t[2] = S.wait_ticks;
    t[3] = (unsigned long long)ran;
  }
}

// Copies records [first, first + cnt) into LDS (the caller synchronizes).
__device__ __forceinline__ void stage_records(const ExecArgs& A, int first, int cnt, DevExec* s_rec, int tid, int nthr) {
  const uint4* src = reinterpret_cast<const uint4*>(A.recs + first);
  uint4* dst = reinterpret_cast<uint4*>(s_rec);
  for (int t = tid; t < cnt * 5; t += nthr) dst[t] = src[t];
}

// One of this rank's buffers by id (selects, so nothing is indexed in memory).
__device__ __forceinline__ unsigned char* buf_of(const WgState& S, uint32_t b) {
  return b == 0u ? S.buf0 : b == 1u ? S.buf1 : S.buf2;
}

// One instruction: slices [s_begin, s_end) of it (s_end < 0: all of them). `first`
// runs its completion waits, `last` sets its completion flag, so an instruction can
// also be run one slice per call (the lazy loop order); `wg_last` marks the
// workgroup's final instruction. OPW >= 0 fixes the low 24 bits of the op word
// (operation and buffers; plan-specialized code), LLK fixes the protocol (-1: the
// launch's). Returns false when the workgroup must leave because a wait gave up.
template <int DT, bool XL, bool NT, long long OPW, int LLK>
__device__ __forceinline__ bool run_instr(const ExecArgs& A, WgState& S, const DevExec& R, int gi, int s_begin,
                                          int s_end, bool first, bool last, bool wg_last) {
  constexpr int esz = Arith<DT>::esz;
  const int tid = S.tid, nthr = S.nthr;
  if (first && S.itrace && tid == 0) S.itrace[4 * size_t(gi)] = (unsigned long long)wall_clock64();
  const uint32_t opw = OPW >= 0 ? (uint32_t(OPW) | (uint32_t(uni(int32_t(R.op))) & 0xff000000u))
                                : uint32_t(uni(int32_t(R.op)));
  const uint32_t op = opw & 15u;
  const int xin = uni(R.xin), xout = uni(R.xout), done_flag = uni(R.done_flag);
  const int nwaits = uni(R.nwaits);
  const int64_t len = uni64(R.len);
  const bool ll = LLK < 0 ? A.ll != 0 : LLK == 1;
  // A receive whose data the sender already placed (direct transport) only waits for
  // the transfer's flag. As the workgroup's final instruction, with no completion flag
  // of its own, nothing depends on that wait: the launch ends only once the sending
  // workgroup has, and the end of the launch makes the sender's stores visible. Its
  // flag round trip would only lengthen the chain, so it is not taken.
  if (wg_last && done_flag < 0 && !ll && (op & OPB_RECV) && !(op & (OPB_DSTA | OPB_SEND))) {
    if (S.itrace && tid == 0 && last) {
      const unsigned long long now = (unsigned long long)wall_clock64();
      S.itrace[4 * size_t(gi) + 1] = now;
      S.itrace[4 * size_t(gi) + 2] = now;
    }
    return true;
  }
  if (first && nwaits > 0) {
    const int wait_begin = uni(R.wait_begin);
    if (tid == 0) {
      int ok = 1;
      for (int w = 0; w < nwaits && ok; ++w)
        ok = wait_geq<true>(&A.dflags[size_t(A.waits[wait_begin + w]) * kFlagStride], A.epoch, A, gi, S.wait_ticks) ? 1 : 0;
      if (!ok) *S.s_abort = 1;
    }
    __syncthreads();
    if (*S.s_abort) return false;
  }
  // The compiler marks every such receive that nothing depends on (OPB_SKIP) wherever
  // it sits: it runs its completion waits (later instructions of the workgroup may be
  // ordered through them), then skips the transfer's flag.
  if (opw & OPB_SKIP) {
    if (S.itrace && tid == 0 && last) {
      const unsigned long long now = (unsigned long long)wall_clock64();
      S.itrace[4 * size_t(gi) + 1] = now;
      S.itrace[4 * size_t(gi) + 2] = now;
    }
    return true;
  }
  // a receive reads its slot, or (direct transport) its own buffer where the sender wrote
  const unsigned char* pa = ((op & OPB_RECV) && !(opw & OPB_LOCAL_IN)) ? S.staging + uni64(R.a_off)
                                                                       : buf_of(S, (opw >> 8) & 3u) + uni64(R.a_off);
  const unsigned char* pb = (op & OPB_SRCB) ? buf_of(S, (opw >> 12) & 3u) + uni64(R.b_off) : nullptr;
  unsigned char* pd = (op & OPB_DSTA) ? buf_of(S, (opw >> 16) & 3u) + uni64(R.d_off) : nullptr;
  unsigned char* pt = nullptr;
  if (op & OPB_SEND) {  // the receiver's slot, or (direct transport) the receiver's buffer
    const uint32_t tb = (opw >> 20) & 15u, tr = opw >> 24;
    pt = (tb == kStagingBuf ? S.staging : tb == 0u ? A.base[0][tr] : tb == 1u ? A.base[1][tr] : A.base[2][tr]) +
         uni64(R.t_off);
  }
  // a send whose receive is skipped sets no flag and need not wait for its stores
  const bool flagged_send = (op & OPB_SEND) && !(opw & OPB_NOFLAG);
  // the receiver's XCD tag: loaded now, first used after this instruction's stores (LL:
  // at its first unit store)
  unsigned long long peer_tag = 0;
  if (XL && flagged_send && A.xcd_tags) {
    const int peer = uni(R.peer_wg);
    if (peer >= 0) peer_tag = __hip_atomic_load(&A.xcd_tags[peer], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // likewise the tag of the one workgroup that waits for this instruction's completion
  unsigned long long done_tag = 0;
  const int done_peer = (XL && last && done_flag >= 0 && A.xcd_tags) ? uni(R.done_peer) : -1;
  if (done_peer >= 0) done_tag = __hip_atomic_load(&A.xcd_tags[done_peer], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (ll) {
    // one pass over the whole range (at s_begin 0); receivers poll the units they consume
    if (s_begin == 0) {
      const WaitCtx wc{A.err, A.abort_word, A.epoch, A.timeout_ticks, gi};
      // Units for a receiver that shares this XCD's L2 are plain stores, any others
      // agent-coherent ones (ll_plain_units), so nothing waits for the stores and no
      // release follows them. Deciding after the stores instead (wait, then release for
      // a receiver elsewhere) made every step wait for its stores, even when no release
      // ran: 8-rank ring launches 0.1-1.1 us slower (32 KiB at k = 1: 18.4 against
      // 17.3 us). A send whose receive is skipped (no flag) has no reader before the
      // launch ends: plain units.
      const unsigned long long here_tag = (XL && flagged_send) ? S.my_tag : 0ull;
      const bool gave_up =
          len > 0 && dispatch_ll<DT, XL>(op, pa, pb, pd, pt, int(len), tid, nthr, A.ll_flag, wc, peer_tag, here_tag);
      // OPB_NOSYNC: nothing later in this workgroup depends on this instruction's local
      // writes or overwrites what it read, so the waves go on without a barrier (up to
      // 1.9 us per 8-rank ring launch at 256 threads); a wave that gave up leaves at once,
      // the launch being aborted already.
      if (opw & OPB_NOSYNC) {
        if (gave_up) return false;
      } else {
        if (gave_up) *S.s_abort = 1;
        __syncthreads();
        if (*S.s_abort) return false;
      }
    }
  } else {
    const int64_t se = A.slice_elems;
    const int nsl = uni(R.nsl);
    const int s_stop = (s_end < 0 || s_end > nsl) ? nsl : s_end;
    for (int s = s_begin; s < s_stop; ++s) {
      const int64_t o = int64_t(s) * se;
      const int n = int((len - o < se) ? (len - o) : se);
      const int64_t bo = o * esz;
      const long long waited =
          dispatch_slice<DT, XL, NT, (OPW >= 0)>(op, (opw & OPB_NOFLAG) != 0, pa + bo, pb ? pb + bo : nullptr, pd ? pd + bo : nullptr,
                                     pt ? pt + bo : nullptr, n, tid, nthr, (op & OPB_RECV) ? &A.xflags[size_t(xin) * kFlagStride] : nullptr,
                                     S.E + (unsigned long long)(s + 1), A, gi);
      if (waited < 0) return false;  // the wait gave up: uniform across the workgroup
      S.wait_ticks += (unsigned long long)waited;
      if (S.itrace && tid == 0 && s == 0) S.itrace[4 * size_t(gi) + 1] = (unsigned long long)wall_clock64();
      if (flagged_send) wait_vm_stores();
      __syncthreads();
      if (flagged_send && tid == 0)
        slot_flag_store<XL>(&A.xflags[size_t(xout) * kFlagStride], S.E + (unsigned long long)(s + 1), XL && use_here(peer_tag) == S.my_tag);
    }
  }
  if (last) {
    if (done_peer >= 0 && use_here(done_tag) == S.my_tag) {
      // The waiter shares this XCD's L2, where this instruction's plain stores land:
      // every wave's stores complete, then a plain flag store (no L2 writeback).
      wait_vm_stores();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(&A.dflags[size_t(done_flag) * kFlagStride], A.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else if (done_flag >= 0 && tid == 0) {
      release_store(&A.dflags[size_t(done_flag) * kFlagStride], A.epoch);
    }
    if (S.itrace && tid == 0) S.itrace[4 * size_t(gi) + 2] = (unsigned long long)wall_clock64();
  }
  return true;
}

// XL: XCD-local layout (every transfer between workgroups whose ids are congruent mod
// 8, which the round-robin dispatch puts on one XCD): transfer data travels with plain
// stores and flags are checked against the receiver's published XCD (slot_flag_store).
// NT: local-buffer loads and local stores carry the non-temporal hint (simple protocol).
template <int DT, bool XL, bool NT>
__global__ __launch_bounds__(1024) void executor_kernel(ExecArgs A) {
  // Set once by any thread that gives up (watchdog, or another workgroup's abort) and
  // never cleared, so a wave that reads it early only leaves a launch that is failing
  // anyway; waves that have ended no longer hold a workgroup barrier.
  __shared__ int s_abort;
  __shared__ DevExec s_rec[kLdsRecs];
  const DevWG W = A.wgs[blockIdx.x];
  if (W.n == 0) return;  // padding id
  WgState S;
  wg_begin<XL>(A, W, S, &s_abort, blockDim.x);
  int ran = 0;
  for (int c0 = 0; c0 < W.n; c0 += kLdsRecs) {
    const int cnt = (W.n - c0 < kLdsRecs) ? (W.n - c0) : kLdsRecs;
    stage_records(A, W.first + c0, cnt, s_rec, S.tid, S.nthr);
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      if (!run_instr<DT, XL, NT, -1, -1>(A, S, s_rec[j], W.first + c0 + j, 0, -1, true, true, c0 + j + 1 == W.n))
        return;
      ++ran;
    }
    if (c0 + kLdsRecs < W.n) __syncthreads();  // all reads of this block done before it is overwritten
  }
  wg_end(A, W, S, ran);
}

}  // namespace
}  // namespace ccl
