// Internal host-side structures of the plan compiler and runtime.
#pragma once

#include <cstdint>
#include <stdexcept>
#include <string>
#include <set>
#include <vector>

#include "../../include/ccl.h"
#include "device_abi.h"

namespace ccl {

struct Error : std::runtime_error {
  int code;
  Error(int c, const std::string& m) : std::runtime_error(m), code(c) {}
};
[[noreturn]] void fail(int code, const std::string& msg);

// Chunk geometry shared by the lowering, byte accounting and the plan checker:
// chunk j covers [floor(j*N/C), floor((j+1)*N/C)); instance i of k takes
// [lo + floor(i*len/k), lo + floor((i+1)*len/k)) of a one-chunk range.
inline int64_t chunk_bound(int64_t j, int64_t N, int64_t C) { return (j * N) / C; }

struct Range {
  int64_t lo = 0, len = 0;
};
// Bound i (0..k) of the k instance pieces of the element range [lo, hi): lo plus
// floor(i (hi - lo) / k) rounded down to a multiple of `align` elements (16 bytes), and
// hi for i = k. Which chain an element follows is decided by its program chunk alone, so
// these bounds change no result. The offsets depend on the range's length only: the
// two ends of a transfer (equal lengths, possibly different 16-byte phases, as an input
// shard and the output) get the same pieces, so their slice flags pair up. When the
// range starts on the 16-byte grid so does every piece (at 8 ranks and 1 MiB, k = 24
// cuts 32,768-element chunks into pieces of 1365.3 elements). A piece is at most
// align - 1 elements longer than ceil((hi - lo) / k).
inline int64_t instance_bound(int i, int k, int64_t lo, int64_t hi, int align) {
  if (i <= 0) return lo;
  if (i >= k) return hi;
  const int64_t f = (int64_t(i) * (hi - lo)) / k;
  return lo + f - f % align;
}
inline Range op_range(int idx, int cnt, int instance, int k, int64_t N, int64_t C, int align) {
  int64_t lo = chunk_bound(idx, N, C), hi = chunk_bound(idx + cnt, N, C);
  if (k > 1) {
    const int64_t a = instance_bound(instance, k, lo, hi, align), b = instance_bound(instance + 1, k, lo, hi, align);
    return {a, b - a};
  }
  return {lo, hi - lo};
}

struct Loc {
  int buf = -1;
  int idx = 0;
  bool valid() const { return buf >= 0; }
  bool operator==(const Loc& o) const { return buf == o.buf && idx == o.idx; }
};

// An instruction of the base program (instance 0), primitive or fused.
struct Instr {
  int rank = 0, channel = 0, cnt = 1;
  bool recv = false;  // first operand is the staging slot of transfer xin
  bool local_in = false;  // direct transport: the received data is written into `a` by the sender
  bool skip = false;      // an idle receive (see mark_idle_receives): not executed
  Loc a, b, d;        // local first operand (if !recv), added operand, local destination
  int xin = -1, xout = -1;
  int chunk_id = 0;
  int pos = 0;        // program position of its first primitive
  // results of scheduling and allocation
  int sp = -1;        // sub-pipeline
  int wg = -1;        // base workgroup
  int done_flag = -1; // base completion-flag id
  std::vector<int> waits;  // base instruction ids whose completion it awaits
  uint32_t opbits() const {
    return (recv ? OPB_RECV : 0u) | (b.valid() ? OPB_SRCB : 0u) | (d.valid() ? OPB_DSTA : 0u) |
           (xout >= 0 ? OPB_SEND : 0u) | (local_in ? OPB_LOCAL_IN : 0u);
  }
};

struct Xfer {
  int src_rank = 0, dst_rank = 0, channel = 0, cnt = 1;
  int sender = -1, receiver = -1;  // base instruction ids
  int phase_idx = -1;
  bool direct = false;  // the sender writes the receiver's destination, no staging slot
  bool noflag = false;  // its receive is skipped: the sender sets no flag
};

struct BaseWG {
  int rank = 0, channel = 0;
  int in_peer = -1, out_peer = -1;
  std::vector<int> instrs;  // execution order
};

struct HostPlan {
  // input
  ccl_program_desc desc{};
  std::vector<ccl_chunk_op> ops;
  int P = 0, C = 0, k = 1;
  int out_chunks = 0, scr_chunks = 0;
  ccl_plan_config cfg{};
  int esz = 4;
  int granule = 1;
  // base program after compilation
  std::vector<Instr> ins;
  std::vector<Xfer> xf;
  std::vector<BaseWG> wgs;
  int num_subpipes = 0;
  int num_done_flags = 0;
  int num_base_waits = 0;
  // lowered tables (all instances)
  std::vector<DevWG> dwg;
  std::vector<DevInstr> dins;
  std::vector<DevXfer> dxf;
  std::vector<int32_t> dwaits;
  std::vector<int> dins_base;  // base instruction id of each lowered instruction
  int64_t staging_bytes = 0;
  int64_t scratch_elems_per_rank = 0;
  int64_t slice_elems = 0;
  int num_connections = 0;
  int max_wg_per_rank = 0;
  int max_resident_wgs = 0;
  int wg_stride = 1;  // lowered ids per base workgroup (>= k; extra ids are empty)
  int dag_width = 0, dag_depth = 0;  // base instruction DAG: maximum antichain, longest chain
  int cu_budget = 0;  // compute units the plan may occupy (0: the whole device)
  double ms[6] = {0, 0, 0, 0, 0, 0};
};

// compiler.cpp
void compile_plan(HostPlan& hp, const ccl_program_desc* prog, int nranks, int nchunks, int k,
                  const ccl_plan_config* cfg);
int64_t output_chunks(const ccl_program_desc& d);
int64_t plan_bytes(const HostPlan& hp, int64_t count);
int64_t output_elems(const HostPlan& hp, int64_t count);
void dag_parallelism(const std::vector<std::set<int>>& succ, int* width, int* depth);
void group_members(const ccl_program_desc& d, int r, std::vector<int>& members, int& pos);
int group_count(const ccl_program_desc& d);

void compute_exec_records(const HostPlan& hp, int64_t count, std::vector<DevExec>& out);

// simulate.cpp
void check_lowered(const HostPlan& hp, uint64_t seed, int nsims);

// executor.hip
// xcd_local: the variant for XCD-local layouts (plain transfer stores, flags checked
// against the receivers' published XCDs); streaming: non-temporal local traffic.
int launch_executor(const ExecArgs& args, int dtype, bool xcd_local, bool streaming, int nwg, int nthreads,
                    void* stream, std::string* err);
int executor_max_blocks_per_cu(int dtype, int nthreads, int* blocks, std::string* err);
int launch_copy_probe(void* dst, const void* src, size_t bytes, int nblocks, int nthreads,
                      void* stream, std::string* err);
int launch_cu_probe(unsigned* out, int nblocks, long long hold_ticks, void* stream, std::string* err);
int launch_hop_probe(unsigned char* data, unsigned char* second, unsigned long long* flags, unsigned long long* tags,
                     long long* ticks, unsigned int* err_words, unsigned long long* abort_word, unsigned long long epoch,
                     long long timeout_ticks, size_t region, size_t rot, int hops, int bytes, int two_operands,
                     int ll, int nthreads, void* stream, std::string* err);
int launch_litmus_mp(unsigned char* data, unsigned long long* flags, unsigned long long* acks,
                     unsigned long long* tags, long long* results, unsigned long long* stop, int npairs, int rounds,
                     int words, int cross, long long timeout_ticks, void* stream, std::string* err);

// static_scratch.hip: the device array behind ccl_execute_static (the entry point that
// allocates nothing). Fixed regions, so that a location only ever holds one kind of
// epoch-valued word whatever plan last used it:
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr size_t kStaticXflagOff = 0, kStaticXflagBytes = size_t(4) << 20;   // 32768 transfer flags
constexpr size_t kStaticDflagOff = kStaticXflagOff + kStaticXflagBytes;
constexpr size_t kStaticDflagBytes = size_t(2) << 20;                        // 16384 completion flags
constexpr size_t kStaticTagOff = kStaticDflagOff + kStaticDflagBytes;
constexpr size_t kStaticTagBytes = size_t(64) << 10;                         // 8192 workgroup XCD tags
constexpr size_t kStaticErrOff = kStaticTagOff + kStaticTagBytes;            // error word (16 B), abort word (8 B)
constexpr size_t kStaticVarOff = kStaticErrOff + 256;                        // tables, records, slots, scratch
constexpr int kMaxDevices = 64;
// Device address of the array on `device` (which must be current on the first call).
int static_scratch_base(int device, unsigned char** base, std::string* err);

// specialize.cpp: plan-specialized kernels (CCL_FLAG_SPECIALIZE / CCL_FLAG_LAZY).
// cus: compute units of the target device; the kernel is compiled for the waves per
// SIMD that the plan's grid needs to be co-resident on them.
// scalar_records: 1 if each step reads its record through the scalar cache, 0 if the
// workgroup stages its records in LDS first.
std::string specialized_source(const HostPlan& hp, bool xcd_local, bool lazy, bool force_loop, int cus,
                               int* num_shapes, int* num_instructions, int* waves_per_simd, int* scalar_records);
int64_t compile_specialized(const std::string& src);  // compile only (no device needed); code bytes
void* load_specialized(const std::string& src, int device, int nthreads, int* blocks_per_cu, int64_t* code_bytes);
int launch_specialized(void* fn, const ExecArgs& args, int nwg, int nthreads, void* stream, std::string* err);

}  // namespace ccl
