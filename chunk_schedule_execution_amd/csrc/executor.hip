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

