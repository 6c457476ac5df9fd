// Plan-specialized executor kernels, generated and compiled when a plan is created.
//
// The interpreting kernel reads every instruction's operation and buffers from its
// record and branches on them. ReSCCL compiles each algorithm's pipelines into a
// kernel of its own instead, so that no instruction stream is parsed at run time
// (ReSCCL report, section 2.2, lightweight kernel generation). Here a plan's
// workgroups are grouped by the sequence of operation words they run (the "shape";
// all instances of a base workgroup share one), and each shape becomes straight-line
// code: one call of the executor's per-instruction step per instruction, with the
// operation and its buffers as template constants. Offsets, lengths and flag indices
// still come from the count-dependent records, so one kernel serves every count.
//
// The lazy variant runs the same code in the other loop order: slice s of every
// instruction before slice s + 1 of any (the whole algorithm once per slice, as an
// interpreter that repeats the algorithm per chunk slice does; ReSCCL report, section
// 2.1, lazy execution), instead of all slices of one instruction before the next.
//
// The device code is the library's own executor source, embedded at build time and
// compiled with hiprtc for gfx950; code objects are cached per source text and
// modules per device for the life of the process.
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <algorithm>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ccl_internal.h"

namespace ccl {

extern const char kEmbeddedExecutorSource[];  // generated at build time

namespace {

// Straight-line code costs about 3.8 KB per instruction; the instruction cache that two
// CUs share holds 64 KB. Measured on ring AllReduce: 15 instructions (52 KB) beat the
// loop form, 23 (87 KB) tie with it, 31 (118 KB) run 1.4x slower at 32 MiB per rank.
constexpr int kMaxStraightInstructions = 24;

// Where the instruction records come from. By default the workgroup copies its records
// into LDS at the start (one vector load per thread, then a barrier) and every step
// reads its fields there. Straight-line code whose pieces are all small reads each
// step's record through the scalar cache instead and skips that start-up copy.
// Measured on the 8-rank ring AllReduce, same plans, both ways: 1.0-1.3 us faster per
// launch for direct-transport pieces of at most 8 KiB (512 KiB direct 21.2 -> 19.9 us,
// 1 MiB k = 16 21.6 -> 20.3), 0.7-1.0 us slower from 10.7 KiB pieces up (2 MiB k = 24
// 27.0 -> 28.0, 3 MiB k = 24 30.1 -> 30.8). Under the LL protocol, whose slots hold twice
// the data, pieces up to 2.7 KiB gained the same (32 - 512 KiB per rank) and 4 KiB ones
// lost (1 MiB k = 32: 23.9 -> 25.1 us).
constexpr int64_t kScalarRecordMaxPiece = 8192;
constexpr int64_t kScalarRecordMaxPieceLL = 3072;

std::string hex32(uint32_t v) {
  char b[16];
  snprintf(b, sizeof b, "0x%06xLL", v);
  return b;
}

struct CodeCache {
  std::mutex mu;
  std::map<std::string, std::vector<char>> code;                   // source -> code object
  std::map<std::pair<std::string, int>, hipFunction_t> functions;  // (source, device) -> kernel
};
CodeCache& cache() {
  static CodeCache* c = new CodeCache();  // never destroyed: modules stay loaded
  return *c;
}

const std::vector<char>& compile_cached(const std::string& src) {
  CodeCache& c = cache();
  {
    std::lock_guard<std::mutex> g(c.mu);
    auto it = c.code.find(src);
    if (it != c.code.end()) return it->second;
  }
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, src.c_str(), "ccl_specialized.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS)
    fail(CCL_ERR_HIP, "hiprtcCreateProgram failed");
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops"};
  const hiprtcResult r = hiprtcCompileProgram(prog, int(sizeof(opts) / sizeof(opts[0])), opts);
  if (r != HIPRTC_SUCCESS) {
    size_t n = 0;
    hiprtcGetProgramLogSize(prog, &n);
    std::string log(n, '\0');
    if (n) hiprtcGetProgramLog(prog, &log[0]);
    hiprtcDestroyProgram(&prog);
    fail(CCL_ERR_HIP, std::string("specialized kernel does not compile: ") + hiprtcGetErrorString(r) + "\n" +
                          log.substr(0, 4000));
  }
  size_t n = 0;
  hiprtcGetCodeSize(prog, &n);
  std::vector<char> obj(n);
  hiprtcGetCode(prog, obj.data());
  hiprtcDestroyProgram(&prog);
  std::lock_guard<std::mutex> g(c.mu);
  return c.code.emplace(src, std::move(obj)).first->second;
}

}  // namespace

// Under the lazy loop order two instructions of one workgroup are ordered slice by
// slice only: slice s of the later one may run before slice s + 1 of the earlier one.
// That keeps their data dependencies only when every local location both touch (one
// of them writing it) is the same chunk range in both, so that their slices cover the
// same elements. Plans where a workgroup writes one range and touches an overlapping
// but different range of the same buffer are refused. (Slots are per transfer and
// direct landings are checked when direct transport is chosen.)
static void check_lazy_local_ranges(const HostPlan& hp) {
  struct Acc {
    int buf, idx, cnt;
    bool write;
  };
  for (const DevWG& G : hp.dwg) {
    std::vector<Acc> seen;
    for (int t = 0; t < G.n; ++t) {
      const DevInstr& D = hp.dins[G.first + t];
      Acc mine[3];
      int n = 0;
      if (!(D.op & OPB_RECV) || (D.op & OPB_LOCAL_IN)) mine[n++] = {D.a_buf, D.a_idx, D.cnt, false};
      if (D.op & OPB_SRCB) mine[n++] = {D.b_buf, D.b_idx, D.cnt, false};
      if (D.op & OPB_DSTA) mine[n++] = {D.d_buf, D.d_idx, D.cnt, true};
      for (int i = 0; i < n; ++i)
        for (const Acc& o : seen) {
          if (o.buf != mine[i].buf || !(o.write || mine[i].write)) continue;
          const bool overlap = o.idx < mine[i].idx + mine[i].cnt && mine[i].idx < o.idx + o.cnt;
          if (overlap && (o.idx != mine[i].idx || o.cnt != mine[i].cnt))
            fail(CCL_ERR_UNSUPPORTED,
                 "the lazy loop order needs the instructions of a workgroup to touch overlapping local ranges only "
                 "as identical chunk ranges (rank " + std::to_string(G.rank) + ", buffer " +
                     std::to_string(o.buf) + ", chunks [" + std::to_string(o.idx) + ", " +
                     std::to_string(o.idx + o.cnt) + ") and [" + std::to_string(mine[i].idx) + ", " +
                     std::to_string(mine[i].idx + mine[i].cnt) + "))");
        }
      for (int i = 0; i < n; ++i) seen.push_back(mine[i]);
    }
  }
}

std::string specialized_source(const HostPlan& hp, bool xcd_local, bool lazy, bool force_loop, int cus,
                               int* num_shapes, int* num_instructions, int* waves_per_simd_out, int* scalar_records) {
  const bool ll = hp.cfg.flags & CCL_FLAG_LL;
  const bool nt = hp.cfg.flags & CCL_FLAG_STREAMING;
  // operation words (operation and buffers, not the peer rank) are count-independent
  std::vector<DevExec> recs;
  compute_exec_records(hp, hp.cfg.max_count, recs);
  const int ngrid = int(hp.dwg.size());
  const int stride = hp.wg_stride;
  const int nbase = (ngrid + stride - 1) / stride;
  std::map<std::vector<uint32_t>, int> shape_of;
  std::vector<std::vector<uint32_t>> shapes;
  std::vector<int> base_shape(nbase, -1);
  int max_n = 1;
  for (int w = 0; w < nbase; ++w) {
    const int g = w * stride;  // instance 0 of base workgroup w
    if (g >= ngrid || hp.dwg[g].n == 0) continue;
    const DevWG& G = hp.dwg[g];
    std::vector<uint32_t> seq(G.n);
    for (int j = 0; j < G.n; ++j) seq[j] = recs[G.first + j].op & 0x00ffffffu;
    for (int i = 1; i < stride && g + i < ngrid; ++i) {  // every instance runs the same operations
      const DevWG& H = hp.dwg[g + i];
      if (H.n == 0) continue;
      if (H.n != G.n) fail(CCL_ERR_INTERNAL, "instances of a workgroup differ in length");
      for (int j = 0; j < H.n; ++j)
        if ((recs[H.first + j].op & 0x00ffffffu) != seq[j]) fail(CCL_ERR_INTERNAL, "instances of a workgroup differ");
    }
    max_n = std::max(max_n, G.n);
    auto it = shape_of.find(seq);
    if (it == shape_of.end()) {
      it = shape_of.emplace(seq, int(shapes.size())).first;
      shapes.push_back(seq);
    }
    base_shape[w] = it->second;
  }
  if (max_n > 512) fail(CCL_ERR_UNSUPPORTED, "specialized kernels hold at most 512 instructions per workgroup");
  // Straight-line code inlines a copy of the per-instruction step (about 3 KB of code)
  // for every instruction of every distinct workgroup program. Measured: up to 24
  // instructions (a 24-rank ring, 80 KB code objects) it beats the interpreter; from
  // about 50 (150 KB and more, beyond the 64 KB instruction cache two CUs share) it
  // loses by 1.3-1.8x. Longer plans get the loop form instead: each workgroup walks its
  // records and switches over the plan's distinct operation words, one inlined step
  // per distinct word (a handful: 3 to 9 in the library's programs).
  size_t total = 0;
  for (const auto& sh : shapes) total += sh.size();
  std::vector<uint32_t> ops;
  for (const auto& sh : shapes)
    for (uint32_t o : sh)
      if (std::find(ops.begin(), ops.end(), o) == ops.end()) ops.push_back(o);
  const bool loop_form = force_loop || total > size_t(kMaxStraightInstructions);
  int64_t max_piece = 0;
  for (const auto& R : recs) max_piece = std::max<int64_t>(max_piece, R.len * hp.esz);
  const bool scalar_recs = !loop_form && !lazy && max_piece <= (ll ? kScalarRecordMaxPieceLL : kScalarRecordMaxPiece);
  if (scalar_records) *scalar_records = scalar_recs ? 1 : 0;
  if (lazy) {
    for (const auto& D : hp.dins)
      if (D.nwaits > 0)
        fail(CCL_ERR_UNSUPPORTED,
             "the lazy loop order needs a plan without cross-workgroup completion waits (one would wait for a "
             "whole instruction while its workgroup is still at an earlier slice of others)");
    if (!(hp.cfg.flags & CCL_FLAG_LL)) check_lazy_local_ranges(hp);
  }
  if (num_shapes) *num_shapes = int(shapes.size());
  if (num_instructions) *num_instructions = int(loop_form ? ops.size() : total);

  const std::string targs = std::to_string(hp.cfg.dtype) + ", " + (xcd_local ? "true" : "false") + ", " +
                            (nt ? "true" : "false");
  const std::string llk = ll ? "1" : "0";
  auto step = [&](uint32_t opw, const std::string& rj, const std::string& gj, const std::string& tail) {
    return "run_instr<" + targs + ", " + hex32(opw) + ", " + llk + ">(A, S, " + rj + ", " + gj + ", " + tail + ")";
  };
  std::string s;
  s += "// generated: plan-specialized executor kernel\n#include <stdint.h>\n";
  s += kEmbeddedExecutorSource;
  s += "\nnamespace ccl {\nnamespace {\n";
  if (scalar_recs) {
    // a record read through a constant-address-space pointer: uniform loads become
    // scalar loads, fields land in scalar registers
    s += "typedef __attribute__((address_space(4))) const DevExec CRec;\n"
         "__device__ __forceinline__ DevExec ld_rec(const CRec* p) {\n"
         "  DevExec r;\n"
         "  r.op = p->op; r.xin = p->xin; r.xout = p->xout; r.done_flag = p->done_flag;\n"
         "  r.wait_begin = p->wait_begin; r.nwaits = p->nwaits; r.nsl = p->nsl; r.peer_wg = p->peer_wg;\n"
         "  r.len = p->len; r.a_off = p->a_off; r.b_off = p->b_off; r.d_off = p->d_off; r.t_off = p->t_off;\n"
         "  r.done_peer = p->done_peer; r.pad1 = 0;\n"
         "  return r;\n}\n";
  }
  if (loop_form) {
    // one step per distinct operation word; j-th record's word selects it
    s += "__device__ __forceinline__ bool spec_step(const ExecArgs& A, WgState& S, const DevExec& R, int gi, int s0, "
         "int s1, bool first, bool last, bool wl) {\n";
    s += "  switch (uint32_t(uni(int32_t(R.op))) & 0xffffffu) {\n";
    for (uint32_t o : ops)
      s += "    case " + hex32(o).substr(0, 8) + "u: return " + step(o, "R", "gi", "s0, s1, first, last, wl") + ";\n";
    s += "    default: return false;  // every word of the plan has a case\n  }\n}\n";
    s += "__device__ __forceinline__ int spec_loop(const ExecArgs& A, WgState& S, const DevExec* r, int g, int n) {\n";
    if (!lazy) {
      s += "  for (int j = 0; j < n; ++j)\n";
      s += "    if (!spec_step(A, S, r[j], g + j, 0, -1, true, true, j + 1 == n)) return -1;\n";
    } else {
      s += "  int iters = 1;\n";
      s += "  for (int j = 0; j < n; ++j) {\n";
      s += std::string("    const int e = ") + (ll ? "1" : "uni(r[j].nsl) > 1 ? uni(r[j].nsl) : 1") + ";\n";
      s += "    iters = iters > e ? iters : e;\n  }\n";
      s += "  for (int it = 0; it < iters; ++it)\n";
      s += "    for (int j = 0; j < n; ++j) {\n";
      s += std::string("      const int e = ") + (ll ? "1" : "uni(r[j].nsl) > 1 ? uni(r[j].nsl) : 1") + ";\n";
      s += "      if (it < e && !spec_step(A, S, r[j], g + j, it, it + 1, it == 0, it == e - 1, j + 1 == n)) return -1;\n";
      s += "    }\n";
    }
    s += "  return n;\n}\n";
  } else {
    s += "__constant__ int kSpecShape[" + std::to_string(std::max(1, nbase)) + "] = {";
    for (int w = 0; w < nbase; ++w) s += (w ? ", " : "") + std::to_string(base_shape[w]);
    if (nbase == 0) s += "-1";
    s += "};\n";
    for (size_t sh = 0; sh < shapes.size(); ++sh) {
      const auto& seq = shapes[sh];
      const int n = int(seq.size());
      s += "__device__ __forceinline__ int spec_shape_" + std::to_string(sh) + "(const ExecArgs& A, WgState& S, " +
           (scalar_recs ? "const CRec* r" : "const DevExec* r") + ", int g) {\n";
      if (!lazy) {
        for (int j = 0; j < n; ++j) {
          const std::string rj = scalar_recs ? "ld_rec(r + " + std::to_string(j) + ")" : "r[" + std::to_string(j) + "]";
          s += "  if (!" +
               step(seq[j], rj, "g + " + std::to_string(j),
                    std::string("0, -1, true, true, ") + (j + 1 == n ? "true" : "false")) +
               ") return -1;\n";
        }
      } else {
        // one slice of every instruction per iteration; an LL instruction is one pass
        s += "  int iters = 1;\n";
        for (int j = 0; j < n; ++j) {
          const std::string e = "e" + std::to_string(j);
          if (ll)
            s += "  const int " + e + " = 1;\n";
          else
            s += "  const int " + e + " = uni(r[" + std::to_string(j) + "].nsl) > 1 ? uni(r[" + std::to_string(j) +
                 "].nsl) : 1;\n";
          s += "  iters = iters > " + e + " ? iters : " + e + ";\n";
        }
        s += "  for (int it = 0; it < iters; ++it) {\n";
        for (int j = 0; j < n; ++j) {
          const std::string e = "e" + std::to_string(j);
          s += "    if (it < " + e + " && !" +
               step(seq[j], "r[" + std::to_string(j) + "]", "g + " + std::to_string(j),
                    "it, it + 1, it == 0, it == " + e + " - 1, " + (j + 1 == n ? "true" : "false")) +
               ") return -1;\n";
        }
        s += "  }\n";
      }
      s += "  return " + std::to_string(n) + ";\n}\n";
    }
  }
  s += "}  // namespace\n}  // namespace ccl\n\n";
  // Every workgroup of the grid must be resident at once (they wait for each other's
  // flags). A grid of more than one workgroup's worth of waves per SIMD asks the
  // compiler for that occupancy (fewer registers per thread) instead of leaving it to
  // the launch bound alone, which lets the register count halve the resident waves.
  const int waves_per_wg = (hp.cfg.nthreads + 63) / 64;
  const int wgs_per_cu = (ngrid + std::max(1, cus) - 1) / std::max(1, cus);
  const int waves_per_simd = std::min(8, (wgs_per_cu * waves_per_wg + 3) / 4);
  if (waves_per_simd_out) *waves_per_simd_out = std::max(1, waves_per_simd);
  s += "extern \"C\" __global__ __launch_bounds__(" + std::to_string(hp.cfg.nthreads) + ")";
  if (waves_per_simd > 1) s += " __attribute__((amdgpu_waves_per_eu(" + std::to_string(waves_per_simd) + ")))";
  s += " void ccl_spec_kernel(ccl::ExecArgs A) {\n";
  s += "  using namespace ccl;\n";
  s += "  __shared__ int s_abort;\n";
  if (!scalar_recs) s += "  __shared__ DevExec s_rec[" + std::to_string(max_n) + "];\n";
  s += "  const DevWG W = A.wgs[blockIdx.x];\n";
  s += "  if (W.n == 0) return;  // padding id\n";
  s += "  WgState S;\n";
  // Straight-line kernels take the workgroup size as a constant, which spares every
  // workgroup the wait for blockDim.x (a load from the implicit kernel arguments): 3 MiB
  // 8-rank ring 30.15 -> 28.9 us, 512 KiB - 2 MiB 1.2-1.4 us faster, large sizes unchanged.
  // The loop form keeps blockDim.x: there the constant changed the compiler's schedule of
  // the reducing steps and cost 16- and 32-rank ring AllReduce 3-9 % (32 MiB, 16 ranks:
  // 378 -> 403 us), while the 2-D ReduceScatter gained 3 % and an 8-rank tree at 64 KiB
  // 0.5 us.
  s += "  wg_begin<" + std::string(xcd_local ? "true" : "false") + ">(A, W, S, &s_abort, " +
       (loop_form ? std::string("int(blockDim.x)") : std::to_string(hp.cfg.nthreads)) + ");\n";
  if (scalar_recs) {
    s += "  const CRec* s_rec = (const CRec*)(A.recs + W.first);\n";
    s += "  __syncthreads();  // s_abort is cleared before any wave can set it\n";
  } else {
    s += "  stage_records(A, W.first, W.n, s_rec, S.tid, S.nthr);\n";
    s += "  __syncthreads();\n";
  }
  s += "  int ran = -1;\n";
  if (loop_form) {
    s += "  ran = spec_loop(A, S, s_rec, W.first, W.n);\n";
  } else {
    s += "  switch (kSpecShape[blockIdx.x / " + std::to_string(stride) + "]) {\n";
    for (size_t sh = 0; sh < shapes.size(); ++sh)
      s += "    case " + std::to_string(sh) + ": ran = spec_shape_" + std::to_string(sh) + "(A, S, s_rec, W.first); break;\n";
    s += "    default: break;\n  }\n";
  }
  s += "  if (ran < 0) return;\n";
  s += "  wg_end(A, W, S, ran);\n}\n";
  return s;
}

int64_t compile_specialized(const std::string& src) { return int64_t(compile_cached(src).size()); }

void* load_specialized(const std::string& src, int device, int nthreads, int* blocks_per_cu, int64_t* code_bytes) {
  const std::vector<char>& obj = compile_cached(src);
  *code_bytes = int64_t(obj.size());
  CodeCache& c = cache();
  hipFunction_t fn = nullptr;
  {
    std::lock_guard<std::mutex> g(c.mu);
    auto it = c.functions.find({src, device});
    if (it != c.functions.end()) fn = it->second;
  }
  if (!fn) {
    hipModule_t mod = nullptr;
    hipError_t e = hipModuleLoadData(&mod, obj.data());
    if (e != hipSuccess) fail(CCL_ERR_HIP, std::string("hipModuleLoadData: ") + hipGetErrorString(e));
    e = hipModuleGetFunction(&fn, mod, "ccl_spec_kernel");
    if (e != hipSuccess) fail(CCL_ERR_HIP, std::string("hipModuleGetFunction: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> g(c.mu);
    c.functions[{src, device}] = fn;
  }
  int b = 0;
  hipError_t e = hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, nthreads, 0);
  if (e != hipSuccess) fail(CCL_ERR_HIP, std::string("occupancy query: ") + hipGetErrorString(e));
  *blocks_per_cu = b;
  return reinterpret_cast<void*>(fn);
}

int launch_specialized(void* fn, const ExecArgs& args, int nwg, int nthreads, void* stream, std::string* err) {
  ExecArgs a = args;
  void* params[] = {&a};
  hipError_t e = hipModuleLaunchKernel(reinterpret_cast<hipFunction_t>(fn), nwg, 1, 1, nthreads, 1, 1, 0,
                                       reinterpret_cast<hipStream_t>(stream), params, nullptr);
  if (e != hipSuccess) {
    *err = std::string("specialized kernel launch: ") + hipGetErrorString(e);
    return CCL_ERR_HIP;
  }
  return CCL_OK;
}

}  // namespace ccl
