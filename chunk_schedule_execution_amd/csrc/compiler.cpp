// Host compiler: chunk program -> verified DAG -> fused instructions -> sub-pipeline
// schedule -> workgroups -> lowered rank x workgroup x pipeline tables.
//
// Steps follow the MSCCLang report, section 3.1 "System design" (tracing and
// dependency analysis into a DAG, instruction generation into send/recv, fusion
// of neighbouring operations into recv-reduce-copy-send, assignment to thread
// blocks by parallelization factor and channel) and the ReSCCL report, section
// 2.1-2.2 (tasks with data and link dependencies, task-level execution,
// hierarchical-priority dynamic scheduling into sub-pipelines, state-based
// thread-block allocation, a rank x block x pipeline layout).
#include <algorithm>
#include <chrono>
#include <cstring>
#include <functional>
#include <map>
#include <numeric>
#include <queue>
#include <set>
#include <tuple>

#include "ccl_internal.h"

namespace ccl {

void fail(int code, const std::string& msg) { throw Error(code, msg); }

namespace {

using Clock = std::chrono::steady_clock;
double ms_since(Clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
}

int64_t gcd64(int64_t a, int64_t b) { return b == 0 ? (a < 0 ? -a : a) : gcd64(b, a % b); }
int64_t lcm64(int64_t a, int64_t b) { return a / gcd64(a, b) * b; }

std::string op_str(const ccl_chunk_op& o) {
  char buf[160];
  snprintf(buf, sizeof buf, "%s(r%d b%d c%d -> r%d b%d c%d x%d ch%d)", o.kind ? "reduce" : "copy", o.src_rank,
           o.src_buf, o.src_idx, o.dst_rank, o.dst_buf, o.dst_idx, o.count, o.channel);
  return buf;
}

// Members of rank r's collective group and r's position in it.
void group_of(const ccl_program_desc& d, int r, std::vector<int>& members, int& pos) {
  int P = d.nranks;
  members.clear();
  if (d.group_scope == CCL_SCOPE_INTRA) {
    int L = d.group_size, g = r / L;
    for (int s = 0; s < L; ++s) members.push_back(g * L + s);
    pos = r % L;
  } else if (d.group_scope == CCL_SCOPE_INTER) {
    int L = d.group_size, l = r % L;
    for (int h = l; h < P; h += L) members.push_back(h);
    pos = r / L;
  } else {
    for (int s = 0; s < P; ++s) members.push_back(s);
    pos = r;
  }
}

int group_n(const ccl_program_desc& d) {
  if (d.group_scope == CCL_SCOPE_INTRA) return d.group_size;
  if (d.group_scope == CCL_SCOPE_INTER) return d.nranks / d.group_size;
  return d.nranks;
}

// ---------------------------------------------------------------- verification

// Chunk-level symbolic execution: every chunk value is a sorted multiset of atoms
// (rank << 16 | chunk) of input chunks; output chunks start as "prior" atoms.
using Atoms = std::vector<uint32_t>;
struct SymVal {
  bool init = false;
  Atoms atoms;
};
constexpr uint32_t kPrior = 0x80000000u;

void verify_postcondition(const HostPlan& hp) {
  const ccl_program_desc& d = hp.desc;
  int P = hp.P, C = hp.C;
  std::vector<std::vector<SymVal>> st[3];
  for (int b = 0; b < 3; ++b) st[b].resize(P);
  for (int r = 0; r < P; ++r) {
    st[0][r].resize(C);
    for (int j = 0; j < C; ++j) st[0][r][j] = {true, {uint32_t(r) << 16 | uint32_t(j)}};
    st[1][r].resize(hp.out_chunks);
    for (int j = 0; j < hp.out_chunks; ++j) st[1][r][j] = {true, {kPrior | uint32_t(r) << 16 | uint32_t(j)}};
    st[2][r].resize(hp.scr_chunks);
  }
  for (const auto& o : hp.ops) {
    for (int t = 0; t < o.count; ++t) {
      const SymVal& s = st[o.src_buf][o.src_rank][o.src_idx + t];
      if (!s.init)
        fail(CCL_ERR_INVALID_PROGRAM, "operation " + op_str(o) + " reads a scratch chunk before it is written");
      SymVal& dv = st[o.dst_buf][o.dst_rank][o.dst_idx + t];
      if (o.kind == CCL_OP_COPY) {
        dv = s;
      } else {
        if (!dv.init)
          fail(CCL_ERR_INVALID_PROGRAM, "operation " + op_str(o) + " reduces into a chunk never written");
        Atoms m;
        std::merge(dv.atoms.begin(), dv.atoms.end(), s.atoms.begin(), s.atoms.end(), std::back_inserter(m));
        dv.atoms.swap(m);
      }
    }
  }
  if (d.collective == CCL_COLL_CUSTOM || (hp.cfg.flags & CCL_FLAG_NO_VERIFY)) return;
  int n = group_n(d);
  std::vector<int> M;
  for (int r = 0; r < P; ++r) {
    int p;
    group_of(d, r, M, p);
    for (int j = 0; j < hp.out_chunks; ++j) {
      Atoms want;
      switch (d.collective) {
        case CCL_COLL_ALLREDUCE:
          for (int m : M) want.push_back(uint32_t(m) << 16 | uint32_t(j));
          break;
        case CCL_COLL_ALLGATHER:
          want.push_back(uint32_t(M[j / C]) << 16 | uint32_t(j % C));
          break;
        case CCL_COLL_REDUCESCATTER: {
          int c = C / n;
          for (int m : M) want.push_back(uint32_t(m) << 16 | uint32_t(p * c + j));
          break;
        }
        case CCL_COLL_ALLTOALL: {
          int c = C / n;
          want.push_back(uint32_t(M[j / c]) << 16 | uint32_t(p * c + j % c));
          break;
        }
        case CCL_COLL_ALLTONEXT:
          want.push_back(p == 0 ? (kPrior | uint32_t(r) << 16 | uint32_t(j)) : (uint32_t(M[p - 1]) << 16 | uint32_t(j)));
          break;
      }
      std::sort(want.begin(), want.end());
      const SymVal& got = st[1][r][j];
      if (got.atoms != want) {
        char buf[200];
        snprintf(buf, sizeof buf, "postcondition fails at rank %d output chunk %d (%zu contributions, want %zu)", r, j,
                 got.atoms.size(), want.size());
        fail(CCL_ERR_INVALID_PROGRAM, buf);
      }
    }
  }
}

void validate(HostPlan& hp, const ccl_program_desc* prog, int nranks, int nchunks, int k,
              const ccl_plan_config* cfg) {
  if (!prog || !cfg) fail(CCL_ERR_INVALID_ARGUMENT, "null program or config");
  const ccl_program_desc& d = *prog;
  if (d.nranks < 1 || d.nranks > kMaxRanks) fail(CCL_ERR_INVALID_ARGUMENT, "nranks must be in [1, 64]");
  if (nranks != d.nranks) fail(CCL_ERR_INVALID_ARGUMENT, "nranks does not match the program");
  if (nchunks != d.in_chunks || nchunks < 1) fail(CCL_ERR_INVALID_ARGUMENT, "nchunks does not match the program's in_chunks");
  if (k < 1 || k > 256) fail(CCL_ERR_INVALID_ARGUMENT, "parallel_factor must be in [1, 256]");
  if (d.nops > 0 && !d.ops) fail(CCL_ERR_INVALID_ARGUMENT, "null ops");
  if (d.collective < CCL_COLL_ALLREDUCE || d.collective > CCL_COLL_CUSTOM) fail(CCL_ERR_UNSUPPORTED, "unknown collective");
  if (d.group_scope != CCL_SCOPE_ALL) {
    if (d.group_scope != CCL_SCOPE_INTRA && d.group_scope != CCL_SCOPE_INTER) fail(CCL_ERR_INVALID_ARGUMENT, "bad group scope");
    if (d.group_size < 1 || d.nranks % d.group_size) fail(CCL_ERR_INVALID_ARGUMENT, "group_size must divide nranks");
  }
  if (cfg->dtype != CCL_F32 && cfg->dtype != CCL_BF16 && cfg->dtype != CCL_I32) fail(CCL_ERR_UNSUPPORTED, "dtype");
  if (cfg->redop != CCL_REDOP_SUM) fail(CCL_ERR_UNSUPPORTED, "only sum is supported");
  if (cfg->max_count < 1) fail(CCL_ERR_INVALID_ARGUMENT, "max_count must be >= 1");
  if (cfg->max_count > (int64_t(1) << 31)) fail(CCL_ERR_INVALID_ARGUMENT, "max_count must be <= 2^31");
  int nt = cfg->nthreads ? cfg->nthreads : 512;
  if (nt < 64 || nt > 1024 || nt % 64) fail(CCL_ERR_INVALID_ARGUMENT, "nthreads must be a multiple of 64 in [64, 1024]");
  if (cfg->slice_bytes < 0) fail(CCL_ERR_INVALID_ARGUMENT, "slice_bytes must be >= 0");
  if (cfg->scheduler < 0 || cfg->scheduler > 2) fail(CCL_ERR_INVALID_ARGUMENT, "scheduler");
  if (cfg->wg_alloc < 0 || cfg->wg_alloc > 1) fail(CCL_ERR_INVALID_ARGUMENT, "wg_alloc");
  if ((cfg->flags & CCL_FLAG_DEBUG_DROP_FLAG) && (cfg->flags & (CCL_FLAG_LL | CCL_FLAG_DIRECT)))
    fail(CCL_ERR_UNSUPPORTED, "flag dropping needs the staged slice-flag protocol (LL flags travel in the data; a "
                              "direct receive at the end of a workgroup is not waited for)");

  hp.desc = d;
  hp.desc.ops = nullptr;
  hp.P = d.nranks;
  hp.C = nchunks;
  hp.k = k;
  hp.cfg = *cfg;
  hp.cfg.nthreads = nt;
  if (hp.cfg.slice_bytes == 0) hp.cfg.slice_bytes = 256 * 1024;
  hp.cu_budget = cfg->num_cus > 0 ? cfg->num_cus : 0;
  if (hp.cfg.num_cus <= 0) hp.cfg.num_cus = 256;
  if (hp.cfg.timeout_us <= 0) hp.cfg.timeout_us = 2000000;
  hp.esz = cfg->dtype == CCL_BF16 ? 2 : 4;
  hp.out_chunks = int(output_chunks(d));
  if (hp.out_chunks < 0) fail(CCL_ERR_INVALID_ARGUMENT, "output chunk count does not fit the collective's shape");
  if (d.collective != CCL_COLL_CUSTOM && d.out_chunks != hp.out_chunks)
    fail(CCL_ERR_INVALID_ARGUMENT, "out_chunks does not match the collective (expected " + std::to_string(hp.out_chunks) + ")");
  if (d.scratch_chunks < 0) fail(CCL_ERR_INVALID_ARGUMENT, "scratch_chunks must be >= 0");
  hp.scr_chunks = d.scratch_chunks;
  hp.ops.assign(d.ops, d.ops + d.nops);

  const int nbuf[3] = {hp.C, hp.out_chunks, hp.scr_chunks};
  int64_t granule = 1;
  for (const auto& o : hp.ops) {
    if (o.kind > CCL_OP_REDUCE) fail(CCL_ERR_INVALID_PROGRAM, "unknown op kind in " + op_str(o));
    if (o.redop != CCL_REDOP_SUM) fail(CCL_ERR_UNSUPPORTED, "reduction op in " + op_str(o));
    if (o.src_rank < 0 || o.src_rank >= hp.P || o.dst_rank < 0 || o.dst_rank >= hp.P)
      fail(CCL_ERR_INVALID_PROGRAM, "rank out of range in " + op_str(o));
    if (o.src_buf < 0 || o.src_buf > 2 || o.dst_buf < 0 || o.dst_buf > 2)
      fail(CCL_ERR_INVALID_PROGRAM, "buffer out of range in " + op_str(o));
    if (o.dst_buf == CCL_BUF_INPUT) fail(CCL_ERR_INVALID_PROGRAM, "programs may not write input buffers: " + op_str(o));
    if (o.count < 1) fail(CCL_ERR_INVALID_PROGRAM, "count must be >= 1 in " + op_str(o));
    if (o.src_idx < 0 || o.src_idx + o.count > nbuf[o.src_buf] || o.dst_idx < 0 || o.dst_idx + o.count > nbuf[o.dst_buf])
      fail(CCL_ERR_INVALID_PROGRAM, "chunk range out of bounds in " + op_str(o));
    if (o.src_rank == o.dst_rank && o.src_buf == o.dst_buf && o.src_idx < o.dst_idx + o.count &&
        o.dst_idx < o.src_idx + o.count)
      fail(CCL_ERR_INVALID_PROGRAM, "source and destination overlap in " + op_str(o));
    // Ranges [a, a+c) and [b, b+c) have equal lengths for every N with N*(a-b) = 0 mod C.
    int64_t diff = std::abs(int64_t(o.src_idx) - int64_t(o.dst_idx)) % hp.C;
    if (diff) granule = lcm64(granule, hp.C / gcd64(hp.C, diff));
  }
  if (d.collective == CCL_COLL_REDUCESCATTER || d.collective == CCL_COLL_ALLTOALL) granule = lcm64(granule, group_n(d));
  if (granule > (int64_t(1) << 30)) fail(CCL_ERR_INVALID_PROGRAM, "chunk offsets force an unusable count granule");
  hp.granule = int(granule);
  // Instances split every chunk separately: a k > 1 plan uses one-chunk operations.
  if (k > 1) {
    std::vector<ccl_chunk_op> ex;
    for (const auto& o : hp.ops)
      for (int t = 0; t < o.count; ++t) {
        ccl_chunk_op e = o;
        e.src_idx += t;
        e.dst_idx += t;
        e.count = 1;
        ex.push_back(e);
      }
    hp.ops.swap(ex);
  }
}

// ---------------------------------------------------------------- DAG + fusion

struct Graph {
  std::vector<std::set<int>> succ, pred;
  void resize(size_t n) {
    succ.assign(n, {});
    pred.assign(n, {});
  }
  void add(int a, int b) {
    if (a == b) return;
    succ[a].insert(b);
    pred[b].insert(a);
  }
};

struct Prim {
  Instr in;
  int d_owner = -1;  // primitive whose write is this node's d (for fused nodes)
};

// Generate primitive instructions (one per local op, send + recv per cross-rank op)
// and their dependency DAG: RAW / WAW / WAR per (rank, buffer, chunk) and send->recv.
void build_primitives(const HostPlan& hp, std::vector<Prim>& prims, std::vector<Xfer>& xf, Graph& g,
                      std::vector<std::vector<int>>& consumers) {
  for (size_t p = 0; p < hp.ops.size(); ++p) {
    const auto& o = hp.ops[p];
    Loc src{o.src_buf, o.src_idx}, dst{o.dst_buf, o.dst_idx};
    Instr base;
    base.channel = o.channel;
    base.cnt = o.count;
    base.chunk_id = o.dst_idx;
    base.pos = int(prims.size());
    if (o.src_rank == o.dst_rank) {
      Instr I = base;
      I.rank = o.src_rank;
      if (o.kind == CCL_OP_COPY) {
        I.a = src;
        I.d = dst;
      } else {
        I.a = dst;
        I.b = src;
        I.d = dst;
      }
      prims.push_back({I, int(prims.size())});
    } else {
      int x = int(xf.size());
      Xfer X;
      X.src_rank = o.src_rank;
      X.dst_rank = o.dst_rank;
      X.channel = o.channel;
      X.cnt = o.count;
      Instr S = base;
      S.rank = o.src_rank;
      S.a = src;
      S.xout = x;
      X.sender = int(prims.size());
      prims.push_back({S, -1});
      Instr R = base;
      R.rank = o.dst_rank;
      R.pos = int(prims.size());
      R.recv = true;
      R.xin = x;
      R.d = dst;
      if (o.kind == CCL_OP_REDUCE) R.b = dst;
      X.receiver = int(prims.size());
      prims.push_back({R, int(prims.size())});
      xf.push_back(X);
    }
  }
  size_t n = prims.size();
  g.resize(n);
  consumers.assign(n, {});
  const int nbuf[3] = {hp.C, hp.out_chunks, hp.scr_chunks};
  // last writer and readers-since-last-write per (rank, buf, chunk)
  std::vector<std::vector<int>> lastw[3];
  std::vector<std::vector<std::vector<int>>> readers[3];
  for (int b = 0; b < 3; ++b) {
    lastw[b].assign(hp.P, std::vector<int>(nbuf[b], -1));
    readers[b].assign(hp.P, std::vector<std::vector<int>>(nbuf[b]));
  }
  for (size_t i = 0; i < n; ++i) {
    const Instr& I = prims[i].in;
    auto read = [&](const Loc& L) {
      for (int c = L.idx; c < L.idx + I.cnt; ++c) {
        int w = lastw[L.buf][I.rank][c];
        if (w >= 0) {
          g.add(w, int(i));
          if (consumers[w].empty() || consumers[w].back() != int(i)) consumers[w].push_back(int(i));
        }
        readers[L.buf][I.rank][c].push_back(int(i));
      }
    };
    if (!I.recv && I.a.valid()) read(I.a);
    if (I.b.valid()) read(I.b);
    if (I.d.valid()) {
      for (int c = I.d.idx; c < I.d.idx + I.cnt; ++c) {
        int w = lastw[I.d.buf][I.rank][c];
        if (w >= 0) g.add(w, int(i));
        for (int r : readers[I.d.buf][I.rank][c]) g.add(r, int(i));
        lastw[I.d.buf][I.rank][c] = int(i);
        readers[I.d.buf][I.rank][c].clear();
      }
    }
    if (I.recv) g.add(xf[I.xin].sender, int(i));
  }
}

// Is there a path a -> ... -> b other than the direct edge?
bool other_path(const Graph& g, int a, int b, std::vector<int>& stamp, int& cur, std::vector<int>& stack) {
  ++cur;
  stack.clear();
  for (int s : g.succ[a])
    if (s != b && stamp[s] != cur) {
      stamp[s] = cur;
      stack.push_back(s);
    }
  while (!stack.empty()) {
    int u = stack.back();
    stack.pop_back();
    if (u == b) return true;
    for (int s : g.succ[u])
      if (stamp[s] != cur) {
        stamp[s] = cur;
        stack.push_back(s);
      }
  }
  return false;
}

void merge_nodes(Graph& g, int x, int y) {
  for (int p : g.pred[y])
    if (p != x) {
      g.succ[p].erase(y);
      g.succ[p].insert(x);
      g.pred[x].insert(p);
    }
  for (int s : g.succ[y]) {
    g.pred[s].erase(y);
    g.pred[s].insert(x);
    g.succ[x].insert(s);
  }
  g.succ[x].erase(y);
  g.succ[y].clear();
  g.pred[y].clear();
}

void remove_node(Graph& g, int x) {
  // keep every ordering that ran through x
  for (int p : g.pred[x]) {
    g.succ[p].erase(x);
    for (int s : g.succ[x]) g.add(p, s);
  }
  for (int s : g.succ[x]) g.pred[s].erase(x);
  g.succ[x].clear();
  g.pred[x].clear();
}

// Fuse value chains and drop dead scratch writes; produces hp.ins / hp.xf and the
// fused DAG (compacted ids).
void fuse(HostPlan& hp, std::vector<std::set<int>>& dag_succ) {
  std::vector<Prim> prims;
  std::vector<Xfer> xf;
  Graph g;
  std::vector<std::vector<int>> consumers;
  build_primitives(hp, prims, xf, g, consumers);
  size_t n = prims.size();
  std::vector<int> group(n), gsize(n, 1);
  std::iota(group.begin(), group.end(), 0);
  std::vector<char> alive(n, 1);
  std::vector<int> stamp(n, 0), stack;
  int cur = 0;
  bool fusion = !(hp.cfg.flags & CCL_FLAG_NO_FUSION);

  for (size_t xi = 0; fusion && xi < n; ++xi) {
    int x = int(xi);
    if (!alive[x] || group[x] != x) continue;
    for (;;) {
      Instr& X = prims[x].in;
      if (!X.d.valid()) break;
      bool merged = false;
      for (int c : consumers[prims[x].d_owner]) {
        if (group[c] != c || gsize[c] != 1 || c == x || !alive[c]) continue;
        const Instr& Y = prims[c].in;
        if (Y.rank != X.rank || Y.channel != X.channel || Y.cnt != X.cnt) continue;
        int rule = 0;
        if (!Y.recv && Y.xout >= 0 && !Y.b.valid() && !Y.d.valid() && Y.a == X.d && X.xout < 0) rule = 1;  // + send
        else if (!Y.recv && Y.b.valid() && Y.a == X.d && Y.d == X.d && !X.b.valid() && X.xout < 0) rule = 2;  // + reduce
        else if (Y.recv && Y.b.valid() && Y.b == X.d && Y.d == X.d && !X.recv && !X.b.valid() && X.xout < 0) rule = 3;
        if (!rule) continue;
        if (other_path(g, x, c, stamp, cur, stack)) continue;
        if (rule == 1) {
          X.xout = Y.xout;
          xf[Y.xout].sender = x;
        } else if (rule == 2) {
          X.b = Y.b;
          prims[x].d_owner = c;
        } else {
          X.recv = true;
          X.xin = Y.xin;
          X.b = X.a;
          X.a = Loc{};
          prims[x].d_owner = c;
          xf[Y.xin].receiver = x;
        }
        merge_nodes(g, x, c);
        group[c] = x;
        gsize[x] += 1;
        alive[c] = 0;
        merged = true;
        break;
      }
      if (!merged) break;
    }
  }
  auto find = [&](int v) {
    while (group[v] != v) v = group[v];
    return v;
  };
  // Dead writes: a scratch value read only inside its own fused instruction.
  if (fusion) {
    for (size_t x = 0; x < n; ++x) {
      if (!alive[x]) continue;
      Instr& X = prims[x].in;
      if (!X.d.valid() || X.d.buf != CCL_BUF_SCRATCH) continue;
      bool outside = false;
      for (int c : consumers[prims[x].d_owner])
        if (find(c) != int(x)) outside = true;
      if (!outside) X.d = Loc{};
    }
  }
  // Remove instructions with no effect (repeat: a dropped receiver drops its send).
  for (bool changed = true; changed;) {
    changed = false;
    for (size_t x = 0; x < n; ++x) {
      if (!alive[x]) continue;
      Instr& X = prims[x].in;
      if (X.d.valid() || X.xout >= 0) continue;
      if (X.recv) {
        int s = xf[X.xin].sender;
        prims[s].in.xout = -1;
        xf[X.xin].sender = xf[X.xin].receiver = -1;
      }
      remove_node(g, int(x));
      alive[x] = 0;
      changed = true;
    }
  }
  // Compact, in program order.
  std::vector<int> newid(n, -1);
  hp.ins.clear();
  for (size_t x = 0; x < n; ++x)
    if (alive[x]) {
      newid[x] = int(hp.ins.size());
      hp.ins.push_back(prims[x].in);
    }
  std::vector<int> xnew(xf.size(), -1);
  hp.xf.clear();
  for (size_t t = 0; t < xf.size(); ++t) {
    if (xf[t].sender < 0 || xf[t].receiver < 0) continue;
    xnew[t] = int(hp.xf.size());
    Xfer X = xf[t];
    X.sender = newid[X.sender];
    X.receiver = newid[X.receiver];
    hp.xf.push_back(X);
  }
  for (auto& I : hp.ins) {
    if (I.xin >= 0) I.xin = xnew[I.xin];
    if (I.xout >= 0) I.xout = xnew[I.xout];
  }
  dag_succ.assign(hp.ins.size(), {});
  for (size_t x = 0; x < n; ++x)
    if (alive[x])
      for (int s : g.succ[x]) dag_succ[newid[x]].insert(newid[s]);
  for (auto& X : hp.xf) {
    if (X.sender < 0 || X.receiver < 0) fail(CCL_ERR_INTERNAL, "transfer lost an endpoint during fusion");
    // where the slot's data sits: same phase as the receiver's destination, else the sender's source
    const Instr& R = hp.ins[X.receiver];
    const Instr& S = hp.ins[X.sender];
    X.phase_idx = R.d.valid() ? R.d.idx : (!S.recv && S.a.valid() ? S.a.idx : -1);
  }
}

// ---------------------------------------------------------------- scheduling

std::vector<int> topo_order(const std::vector<std::set<int>>& succ, const std::vector<int>& key) {
  size_t n = succ.size();
  std::vector<int> indeg(n, 0), order;
  for (size_t u = 0; u < n; ++u)
    for (int v : succ[u]) indeg[v]++;
  std::priority_queue<std::pair<int, int>, std::vector<std::pair<int, int>>, std::greater<>> q;
  for (size_t u = 0; u < n; ++u)
    if (!indeg[u]) q.push({key[u], int(u)});
  while (!q.empty()) {
    int u = q.top().second;
    q.pop();
    order.push_back(u);
    for (int v : succ[u])
      if (--indeg[v] == 0) q.push({key[v], v});
  }
  if (order.size() != n) fail(CCL_ERR_INTERNAL, "dependency graph has a cycle");
  return order;
}

// Task link: the connection its send occupies (src rank, dst rank, channel); -1 if none.
int64_t link_of(const HostPlan& hp, const Instr& I) {
  if (I.xout < 0) return -1;
  const Xfer& X = hp.xf[I.xout];
  return (int64_t(X.src_rank) * kMaxRanks + X.dst_rank) * 65536 + X.channel;
}

// ---------------------------------------------------------------- direct transport

// A receive that only copies the incoming data into a local location (and perhaps
// forwards it) can have the sender write that location itself, with no staging slot,
// when no instruction of the receiving rank that could run before the receive touches
// the location: every other accessor must be a descendant of the receive in the DAG.
// The receive then waits for the transfer's flag and reads (forwards) from there.
// Direct transport: the sender writes the received data straight into a location of
// the receiving rank (its landing), so the transfer needs no staging slot. The landing
// is the receive's destination; a receive that reduces without storing locally (it only
// forwards the sum) lands in the same chunk of the rank's output, else of its scratch.
// Legal when every other instruction of that rank that touches the landing is either a
// DAG descendant of the receive (it runs after the data was consumed) or a DAG ancestor
// of the sender (it is done with it before the sender writes), and touches exactly the
// landing's chunk range if the DAG orders it only slice by slice. Every DAG edge is
// enforced at run time: program order and completion flags order a whole instruction
// before the next, but a transfer (and program order under the lazy loop order) only
// orders slice s after slice s. Along a path of such edges alone, slice s of one end
// comes before slice s of the other, which covers the same elements only when both
// operate on the same range. A copy-only receive then only waits (and forwards from its
// landing); a reducing one reads its landing in place of the slot.
void choose_direct(HostPlan& hp, const std::vector<std::set<int>>& dag) {
  if (!(hp.cfg.flags & CCL_FLAG_DIRECT) || (hp.cfg.flags & CCL_FLAG_LL)) return;
  const size_t n = hp.ins.size();
  std::vector<std::vector<int>> pred(n);
  for (size_t u = 0; u < n; ++u)
    for (int v : dag[u]) pred[v].push_back(int(u));
  std::vector<int> below(n, -1), above(n, -1), stack;
  // transfer chains: the instruction a sender feeds and the one a receiver is fed by
  std::vector<int> feeds(n, -1), fed_by(n, -1);
  for (const Xfer& X : hp.xf) {
    feeds[X.sender] = X.receiver;
    fed_by[X.receiver] = X.sender;
  }
  const bool lazy = (hp.cfg.flags & CCL_FLAG_LAZY) != 0;
  std::vector<int> slicewise(n, -1);
  auto overlaps = [](const Loc& l, int lc, const Loc& m, int mc) {
    return l.valid() && m.valid() && l.buf == m.buf && l.idx < m.idx + mc && m.idx < l.idx + lc;
  };
  auto mark_from = [&](int root, int tag, std::vector<int>& mark, bool down) {
    stack.assign(1, root);
    mark[root] = tag;
    while (!stack.empty()) {
      int u = stack.back();
      stack.pop_back();
      const auto visit = [&](int v) {
        if (mark[v] != tag) {
          mark[v] = tag;
          stack.push_back(v);
        }
      };
      if (down)
        for (int v : dag[u]) visit(v);
      else
        for (int v : pred[u]) visit(v);
    }
  };
  for (size_t x = 0; x < hp.xf.size(); ++x) {
    Xfer& X = hp.xf[x];
    Instr& R = hp.ins[X.receiver];
    if (!R.recv || R.local_in || hp.ins[X.sender].rank == R.rank) continue;
    std::vector<Loc> cands;
    if (R.d.valid()) {
      cands.push_back(R.d);
    } else if (R.b.valid()) {
      if (R.b.idx + R.cnt <= hp.out_chunks) cands.push_back(Loc{CCL_BUF_OUTPUT, R.b.idx});
      if (R.b.idx + R.cnt <= hp.scr_chunks) cands.push_back(Loc{CCL_BUF_SCRATCH, R.b.idx});
    }
    if (cands.empty()) continue;
    mark_from(X.receiver, int(x), below, true);
    mark_from(X.sender, int(x), above, false);
    for (const Loc& land : cands) {
      if (R.b.valid() && overlaps(land, R.cnt, R.b, R.cnt)) continue;  // the operand is read as data lands
      bool ok = true;
      for (size_t i = 0; i < n && ok; ++i) {
        if (below[i] == int(x) || above[i] == int(x)) continue;
        const Instr& I = hp.ins[i];
        if (I.rank != R.rank) continue;
        if (overlaps(I.a, I.cnt, land, R.cnt) || overlaps(I.b, I.cnt, land, R.cnt) ||
            overlaps(I.d, I.cnt, land, R.cnt))
          ok = false;
      }
      // instructions ordered against the transfer only slice by slice
      for (int u = feeds[X.receiver]; u >= 0 && slicewise[u] != int(x); u = feeds[u]) slicewise[u] = int(x);
      for (int u = X.sender; u >= 0 && slicewise[u] != int(x); u = fed_by[u]) slicewise[u] = int(x);
      for (size_t i = 0; i < n && ok; ++i) {
        if (i == size_t(X.receiver) || (below[i] != int(x) && above[i] != int(x))) continue;
        if (!lazy && slicewise[i] != int(x)) continue;
        const Instr& I = hp.ins[i];
        if (I.rank != R.rank) continue;
        for (const Loc* l : {&I.a, &I.b, &I.d})
          if (overlaps(*l, I.cnt, land, R.cnt) && !(l->buf == land.buf && l->idx == land.idx && I.cnt == R.cnt))
            ok = false;  // ordered by the DAG, but its slices cover other elements
      }
      if (!ok) continue;
      X.direct = true;
      R.local_in = true;
      R.a = land;
      if (!R.b.valid()) R.d = Loc{};  // copy-only: the data is already in place
      break;
    }
  }
}

void schedule(HostPlan& hp, const std::vector<std::set<int>>& succ) {
  size_t n = hp.ins.size();
  std::vector<int> pos(n);
  for (size_t i = 0; i < n; ++i) pos[i] = hp.ins[i].pos;
  std::vector<int> order = topo_order(succ, pos);
  if (hp.cfg.scheduler == CCL_SCHED_PROGRAM_ORDER) {
    for (size_t t = 0; t < n; ++t) hp.ins[order[t]].sp = int(t);
    hp.num_subpipes = int(n);
    return;
  }
  // depth = longest path from a source
  std::vector<int> depth(n, 0), indeg(n, 0);
  for (int u : order)
    for (int v : succ[u]) depth[v] = std::max(depth[v], depth[u] + 1);
  for (size_t u = 0; u < n; ++u)
    for (int v : succ[u]) indeg[v]++;
  // tasks grouped by chunk id, each list ordered by (depth, id)
  std::map<int, std::vector<int>> by_chunk_map;
  for (size_t i = 0; i < n; ++i) by_chunk_map[hp.ins[i].chunk_id].push_back(int(i));
  std::vector<std::vector<int>> by_chunk;
  for (auto& kv : by_chunk_map) {
    auto v = kv.second;
    std::sort(v.begin(), v.end(), [&](int a, int b) { return std::tie(depth[a], a) < std::tie(depth[b], b); });
    by_chunk.push_back(v);
  }
  size_t nc = by_chunk.size();
  std::vector<int> done_preds(n, 0), prio(nc, 0), head(nc, 0);
  std::vector<int64_t> link(n);
  for (size_t i = 0; i < n; ++i) link[i] = link_of(hp, hp.ins[i]);
  size_t remaining = n;
  int s = 0;
  std::vector<int> admitted;
  while (remaining) {
    admitted.clear();
    std::set<int64_t> used;
    auto ready = [&](int t) { return hp.ins[t].sp < 0 && done_preds[t] == indeg[t]; };
    if (hp.cfg.scheduler == CCL_SCHED_HPDS) {
      // Repeatedly: the chunk executed least so far (ties: lower id) that has a
      // ready task whose link is still free in this sub-pipeline gets one task in.
      for (;;) {
        int best_c = -1, best_t = -1;
        for (size_t c = 0; c < nc; ++c) {
          if (best_c >= 0 && prio[c] >= prio[best_c]) continue;
          while (head[c] < int(by_chunk[c].size()) && hp.ins[by_chunk[c][head[c]]].sp >= 0) head[c]++;
          for (int idx = head[c]; idx < int(by_chunk[c].size()); ++idx) {
            int t = by_chunk[c][idx];
            if (!ready(t)) continue;
            if (link[t] >= 0 && used.count(link[t])) continue;
            best_c = int(c);
            best_t = t;
            break;
          }
        }
        if (best_t < 0) break;
        hp.ins[best_t].sp = s;
        if (link[best_t] >= 0) used.insert(link[best_t]);
        prio[best_c]++;
        admitted.push_back(best_t);
      }
    } else {
      // Round robin: every chunk in id order puts its next ready task in; links unchecked.
      for (size_t c = 0; c < nc; ++c) {
        for (int t : by_chunk[c])
          if (ready(t)) {
            hp.ins[t].sp = s;
            admitted.push_back(t);
            break;
          }
      }
    }
    if (admitted.empty()) fail(CCL_ERR_INTERNAL, "scheduler made no progress");
    for (int t : admitted)
      for (int v : succ[t]) done_preds[v]++;
    remaining -= admitted.size();
    ++s;
  }
  hp.num_subpipes = s;
}

// ---------------------------------------------------------------- workgroups

void allocate_workgroups(HostPlan& hp) {
  size_t n = hp.ins.size();
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    return std::tie(hp.ins[a].sp, hp.ins[a].pos) < std::tie(hp.ins[b].sp, hp.ins[b].pos);
  });
  hp.wgs.clear();
  std::map<std::pair<int, int>, std::vector<int>> at;  // (rank, channel) -> wg ids
  for (int t : order) {
    Instr& I = hp.ins[t];
    int in = I.xin >= 0 ? hp.xf[I.xin].src_rank : -1;
    int out = I.xout >= 0 ? hp.xf[I.xout].dst_rank : -1;
    auto& cands = at[{I.rank, I.channel}];
    int pick = -1, best = -1;
    for (int w : cands) {
      BaseWG& W = hp.wgs[w];
      bool ok_in = in < 0 || W.in_peer < 0 || W.in_peer == in;
      bool ok_out = out < 0 || W.out_peer < 0 || W.out_peer == out;
      if (!ok_in || !ok_out) continue;
      int score = (in >= 0 && W.in_peer == in) + (out >= 0 && W.out_peer == out);
      if (score > best) {
        best = score;
        pick = w;
      }
    }
    if (pick < 0) {
      pick = int(hp.wgs.size());
      BaseWG W;
      W.rank = I.rank;
      W.channel = I.channel;
      hp.wgs.push_back(W);
      cands.push_back(pick);
    }
    BaseWG& W = hp.wgs[pick];
    if (in >= 0) W.in_peer = in;
    if (out >= 0) W.out_peer = out;
    W.instrs.push_back(t);
    I.wg = pick;
  }
  if (hp.cfg.wg_alloc == CCL_WG_STATE) {
    // Merge workgroups of one rank whose sets of active sub-pipelines are disjoint,
    // first fit in order of first activation.
    std::vector<std::set<int>> act(hp.wgs.size());
    for (size_t w = 0; w < hp.wgs.size(); ++w)
      for (int t : hp.wgs[w].instrs) act[w].insert(hp.ins[t].sp);
    std::vector<int> worder(hp.wgs.size());
    std::iota(worder.begin(), worder.end(), 0);
    std::sort(worder.begin(), worder.end(), [&](int a, int b) {
      return std::tie(*act[a].begin(), a) < std::tie(*act[b].begin(), b);
    });
    std::vector<BaseWG> merged;
    std::vector<std::set<int>> macts;
    for (int w : worder) {
      int into = -1;
      for (size_t m = 0; m < merged.size() && into < 0; ++m) {
        if (merged[m].rank != hp.wgs[w].rank) continue;
        bool disjoint = true;
        for (int s : act[w])
          if (macts[m].count(s)) {
            disjoint = false;
            break;
          }
        if (disjoint) into = int(m);
      }
      if (into < 0) {
        into = int(merged.size());
        BaseWG W = hp.wgs[w];
        W.instrs.clear();
        merged.push_back(W);
        macts.push_back({});
      }
      for (int t : hp.wgs[w].instrs) merged[into].instrs.push_back(t);
      macts[into].insert(act[w].begin(), act[w].end());
    }
    hp.wgs.swap(merged);
  }
  // execution order inside a workgroup: sub-pipeline, then program position
  for (size_t w = 0; w < hp.wgs.size(); ++w) {
    auto& v = hp.wgs[w].instrs;
    std::sort(v.begin(), v.end(), [&](int a, int b) {
      return std::tie(hp.ins[a].sp, hp.ins[a].pos) < std::tie(hp.ins[b].sp, hp.ins[b].pos);
    });
    for (int t : v) hp.ins[t].wg = int(w);
  }
  // workgroups ordered by rank, then first task
  std::vector<int> word(hp.wgs.size());
  std::iota(word.begin(), word.end(), 0);
  std::stable_sort(word.begin(), word.end(), [&](int a, int b) { return hp.wgs[a].rank < hp.wgs[b].rank; });
  std::vector<BaseWG> sorted;
  for (int w : word) sorted.push_back(hp.wgs[w]);
  hp.wgs.swap(sorted);
  for (size_t w = 0; w < hp.wgs.size(); ++w)
    for (int t : hp.wgs[w].instrs) hp.ins[t].wg = int(w);
}

// Cross-workgroup waits. Edges: sequence (next instruction of a workgroup starts after
// the previous one completes), transfer (receiver's slice s after sender's slice s, so
// the receiver completes after the sender), data (same rank, needs start-after-complete).
// A data edge u->v across workgroups gets a completion wait unless some path already
// makes v start after u completes.
void compute_waits(HostPlan& hp, const std::vector<std::set<int>>& dag) {
  size_t n = hp.ins.size();
  std::vector<std::vector<int>> seq(n), xfe(n), data(n);
  std::vector<int> prev_in_wg(n, -1);
  for (const auto& W : hp.wgs)
    for (size_t i = 1; i < W.instrs.size(); ++i) {
      seq[W.instrs[i - 1]].push_back(W.instrs[i]);
      prev_in_wg[W.instrs[i]] = W.instrs[i - 1];
    }
  for (const auto& X : hp.xf) xfe[X.sender].push_back(X.receiver);
  std::vector<std::set<int>> all(n);
  for (size_t u = 0; u < n; ++u) {
    for (int v : dag[u]) {
      all[u].insert(v);
      if (hp.ins[u].rank == hp.ins[v].rank) data[u].push_back(v);
    }
    for (int v : seq[u]) all[u].insert(v);
  }
  std::vector<int> pos(n);
  for (size_t i = 0; i < n; ++i) pos[i] = hp.ins[i].pos;
  std::vector<int> order;
  try {
    order = topo_order(all, pos);
  } catch (const Error&) {
    fail(CCL_ERR_INTERNAL, "workgroup order contradicts the dependency graph (would deadlock)");
  }
  std::vector<int> topo_idx(n);
  for (size_t i = 0; i < n; ++i) topo_idx[order[i]] = int(i);
  size_t words = (n + 63) / 64;
  std::vector<uint64_t> S(n * words, 0);  // S(u): nodes that start after u completes
  auto set_bit = [&](size_t u, int v) { S[u * words + v / 64] |= uint64_t(1) << (v % 64); };
  auto has_bit = [&](size_t u, int v) { return (S[u * words + v / 64] >> (v % 64)) & 1; };
  auto or_into = [&](size_t u, size_t w) {
    for (size_t i = 0; i < words; ++i) S[u * words + i] |= S[w * words + i];
  };
  for (auto& I : hp.ins) I.waits.clear();
  for (size_t ri = n; ri-- > 0;) {
    int u = order[ri];
    for (int w : seq[u]) {
      set_bit(u, w);
      or_into(u, w);
    }
    for (int w : xfe[u]) or_into(u, w);
    std::vector<int> dv = data[u];
    std::sort(dv.begin(), dv.end(), [&](int a, int b) { return topo_idx[a] < topo_idx[b]; });
    for (int v : dv) {
      if (hp.ins[v].wg == hp.ins[u].wg) {
        // same workgroup: its order must already put u first
        if (topo_idx[u] > topo_idx[v]) fail(CCL_ERR_INTERNAL, "workgroup order breaks a dependency");
        continue;
      }
      if (has_bit(u, v)) continue;
      hp.ins[v].waits.push_back(u);
      set_bit(u, v);
      or_into(u, v);
    }
  }
  hp.num_done_flags = 0;
  hp.num_base_waits = 0;
  for (auto& I : hp.ins) I.done_flag = -1;
  for (auto& I : hp.ins)
    for (int u : I.waits) {
      if (hp.ins[u].done_flag < 0) hp.ins[u].done_flag = hp.num_done_flags++;
      hp.num_base_waits++;
    }
}

// A receive of direct transport whose data the sender writes into its place, that
// stores nothing itself, forwards nothing, sets no completion flag and precedes no other
// instruction in the dependency graph only delays its workgroup: nothing observes its
// wait before the launch ends, and the end of the launch makes the sender's stores
// visible. It is skipped, and its sender neither waits for its store acknowledgements
// nor sets the transfer's flag (a bubble per slice on long copies).
void mark_idle_receives(HostPlan& hp, const std::vector<std::set<int>>& dag) {
  for (auto& X : hp.xf) X.noflag = false;
  for (size_t t = 0; t < hp.ins.size(); ++t) {
    Instr& I = hp.ins[t];
    I.skip = I.recv && I.local_in && !I.b.valid() && !I.d.valid() && I.xout < 0 && I.done_flag < 0 && dag[t].empty();
    if (I.skip) hp.xf[I.xin].noflag = true;
  }
}

// ---------------------------------------------------------------- lowering

int len_idx_of(const HostPlan& hp, int t, int depth = 0) {
  const Instr& I = hp.ins[t];
  if ((!I.recv || I.local_in) && I.a.valid()) return I.a.idx;
  if (I.d.valid()) return I.d.idx;
  if (I.b.valid()) return I.b.idx;
  if (I.recv && depth < 1024) return len_idx_of(hp, hp.xf[I.xin].sender, depth + 1);
  fail(CCL_ERR_INTERNAL, "instruction without a chunk range");
}

// Under LL a workgroup's waves only need a barrier after an instruction when a later
// instruction of the same workgroup touches a local chunk range it writes, or writes a
// range it reads: those accesses may use another thread-to-element mapping. The check
// runs on chunk indices, so it holds for every count; a range whose length is another
// chunk's is widened by one chunk at its end, since ragged counts give chunks different
// lengths.
// Inputs and outputs are separate buffers (out of place), the scratch buffer a third.
// An instruction that sets a completion flag keeps its barrier: the flag follows the
// stores of every wave.
static void mark_unsynced(HostPlan& hp) {
  struct Acc {
    int buf, lo, hi;  // chunk indices [lo, hi)
  };
  auto accesses = [&](const DevInstr& D, std::vector<Acc>& rd, std::vector<Acc>& wr) {
    rd.clear();
    wr.clear();
    // the element range's length is that of chunk pad0: at another chunk's offset it may
    // run past that chunk's end by less than a chunk
    auto acc = [&](int buf, int idx) { return Acc{buf, idx, idx + D.cnt + (idx == D.pad0 ? 0 : 1)}; };
    if (!(D.op & OPB_RECV) || (D.op & OPB_LOCAL_IN)) rd.push_back(acc(D.a_buf, D.a_idx));
    if (D.op & OPB_SRCB) rd.push_back(acc(D.b_buf, D.b_idx));
    if (D.op & OPB_DSTA) wr.push_back(acc(D.d_buf, D.d_idx));
  };
  auto meet = [](const std::vector<Acc>& x, const std::vector<Acc>& y) {
    for (const Acc& a : x)
      for (const Acc& b : y)
        if (a.buf == b.buf && a.lo < b.hi && b.lo < a.hi) return true;
    return false;
  };
  std::vector<Acc> ri, wi, rj, wj;
  for (const DevWG& G : hp.dwg) {
    for (int i = G.first; i < G.first + G.n; ++i) {
      DevInstr& D = hp.dins[i];
      if (D.done_flag >= 0) continue;
      accesses(D, ri, wi);
      bool hazard = false;
      for (int j = i + 1; j < G.first + G.n && !hazard; ++j) {
        accesses(hp.dins[j], rj, wj);
        hazard = meet(wi, rj) || meet(wi, wj) || meet(ri, wj);
      }
      if (!hazard) D.op |= OPB_NOSYNC;
    }
  }
}

void lower(HostPlan& hp) {
  int k = hp.k;
  int nW = int(hp.wgs.size()), nX = int(hp.xf.size()), nD = hp.num_done_flags;
  (void)nD;
  hp.dwg.clear();
  hp.dins.clear();
  hp.dxf.assign(size_t(nX) * k, DevXfer{});
  // the base workgroup that waits for each instruction's completion flag, if only one does
  std::vector<int> waiter_wg(hp.ins.size(), -1);
  {
    std::vector<char> several(hp.ins.size(), 0);
    for (const auto& V : hp.ins)
      for (int u : V.waits) {
        if (waiter_wg[u] >= 0 && waiter_wg[u] != V.wg) several[u] = 1;
        waiter_wg[u] = V.wg;
      }
    for (size_t u = 0; u < hp.ins.size(); ++u)
      if (several[u]) waiter_wg[u] = -1;
  }
  hp.dwaits.clear();
  hp.dins_base.clear();
  int64_t M = hp.cfg.max_count;
  // staging slots, one per transfer and instance, sized for max_count
  int64_t off = 0;
  for (int x = 0; x < nX; ++x) {
    const Xfer& X = hp.xf[x];
    // k > 1: a piece is at most ceil(chunk / k) plus 16 bytes' worth of elements (its
    // bounds are rounded to the 16-byte grid)
    int64_t cap = (k == 1) ? (int64_t(X.cnt) * M) / hp.C + 2 : (M / hp.C + 2) / k + 2 + 16 / hp.esz;
    int64_t bytes = ((cap + 16) * hp.esz + 255) / 256 * 256;
    if (hp.cfg.flags & CCL_FLAG_LL) bytes *= 2;  // every 4 data bytes travel with a 4-byte flag
    if (X.direct) bytes = 0;                     // written straight into the receiver's buffer
    for (int i = 0; i < k; ++i) {
      DevXfer& D = hp.dxf[size_t(x) * k + i];
      D.slot_off = uint64_t(off);
      D.phase_idx = X.phase_idx;
      D.instance = i;
      D.cnt = X.cnt;
      D.direct = X.direct ? 1 : 0;
      off += bytes;
    }
  }
  hp.staging_bytes = off;
  bool uses_scratch = false;
  for (auto& I : hp.ins)
    if (I.a.buf == CCL_BUF_SCRATCH || I.b.buf == CCL_BUF_SCRATCH || I.d.buf == CCL_BUF_SCRATCH) uses_scratch = true;
  hp.scratch_elems_per_rank = uses_scratch ? chunk_bound(hp.scr_chunks, M, hp.C) + 64 : 0;
  std::vector<int> per_rank(hp.P, 0);
  // Lowered workgroup (w, i) gets id w*stride + i. Workgroups are dispatched to the
  // eight XCDs round robin by id, so with a stride that is a multiple of 8 every
  // instance keeps all its workgroups -- the ones that hand slots to each other -- on
  // one XCD (i mod 8). Padding ids run no instructions; padding is used only when the
  // padded grid still fits a conservative residency estimate.
  int stride = k;
  const int padded = (k + 7) / 8 * 8;
  const int est_resident = hp.cfg.num_cus * std::max(1, 1024 / hp.cfg.nthreads);
  if (padded != k && int64_t(nW) * padded <= est_resident) stride = padded;
  hp.wg_stride = stride;
  for (int w = 0; w < nW; ++w) {
    const BaseWG& W = hp.wgs[w];
    per_rank[W.rank] += k;
    for (int i = 0; i < stride; ++i) {
      if (i >= k) {
        DevWG E{W.rank, int(hp.dins.size()), 0, int(hp.dwg.size())};
        hp.dwg.push_back(E);
        continue;
      }
      DevWG G;
      G.rank = W.rank;
      G.first = int(hp.dins.size());
      G.n = int(W.instrs.size());
      G.trace_slot = int(hp.dwg.size());
      for (int t : W.instrs) {
        const Instr& I = hp.ins[t];
        DevInstr D{};
        D.op = I.opbits() | (I.skip ? OPB_SKIP : 0u) | (I.xout >= 0 && hp.xf[I.xout].noflag ? OPB_NOFLAG : 0u);
        D.cnt = I.cnt;
        D.a_buf = I.a.buf;
        D.a_idx = I.a.idx;
        D.b_buf = I.b.buf;
        D.b_idx = I.b.idx;
        D.d_buf = I.d.buf;
        D.d_idx = I.d.idx;
        D.xin = I.xin >= 0 ? I.xin * k + i : -1;
        D.xout = I.xout >= 0 ? I.xout * k + i : -1;
        D.wait_begin = int(hp.dwaits.size());
        D.nwaits = int(I.waits.size());
        for (int u : I.waits) hp.dwaits.push_back(hp.ins[u].done_flag * k + i);
        D.done_flag = I.done_flag >= 0 ? I.done_flag * k + i : -1;
        D.instance = i;
        D.pad0 = len_idx_of(hp, t);
        D.peer_wg = I.xout >= 0 ? hp.ins[hp.xf[I.xout].receiver].wg * stride + i : -1;
        D.done_peer = I.done_flag >= 0 && waiter_wg[t] >= 0 ? waiter_wg[t] * stride + i : -1;
        D.t_buf = D.t_rank = D.t_idx = -1;
        if (I.xout >= 0 && hp.xf[I.xout].direct) {
          const Instr& R = hp.ins[hp.xf[I.xout].receiver];
          D.t_buf = R.a.buf;
          D.t_rank = R.rank;
          D.t_idx = R.a.idx;
        }
        hp.dins.push_back(D);
        hp.dins_base.push_back(t);
      }
      hp.dwg.push_back(G);
    }
  }
  hp.max_wg_per_rank = 0;
  for (int r = 0; r < hp.P; ++r) hp.max_wg_per_rank = std::max(hp.max_wg_per_rank, per_rank[r]);
  std::set<std::tuple<int, int, int>> conns;
  for (auto& X : hp.xf) conns.insert({X.src_rank, X.dst_rank, X.channel});
  hp.num_connections = int(conns.size()) * k;
  int64_t se = hp.cfg.slice_bytes / hp.esz;
  se = se / 64 * 64;
  hp.slice_elems = std::max<int64_t>(se, 64);
  if (hp.cfg.flags & CCL_FLAG_LL) mark_unsynced(hp);
}

}  // namespace

int64_t output_chunks(const ccl_program_desc& d) {
  int P = d.nranks, C = d.in_chunks;
  int n = (d.group_scope == CCL_SCOPE_INTRA) ? d.group_size : (d.group_scope == CCL_SCOPE_INTER ? P / std::max(1, d.group_size) : P);
  switch (d.collective) {
    case CCL_COLL_ALLREDUCE:
    case CCL_COLL_ALLTOALL:
    case CCL_COLL_ALLTONEXT:
      return C;
    case CCL_COLL_ALLGATHER:
      return int64_t(n) * C;
    case CCL_COLL_REDUCESCATTER:
      return (n > 0 && C % n == 0) ? C / n : -1;
    case CCL_COLL_CUSTOM:
      return d.out_chunks;
  }
  return -1;
}

void group_members(const ccl_program_desc& d, int r, std::vector<int>& members, int& pos) { group_of(d, r, members, pos); }
int group_count(const ccl_program_desc& d) { return group_n(d); }

int64_t output_elems(const HostPlan& hp, int64_t count) { return chunk_bound(hp.out_chunks, count, hp.C); }

int64_t plan_bytes(const HostPlan& hp, int64_t count) {
  int64_t total = 0;
  for (size_t j = 0; j < hp.dins.size(); ++j) {
    const DevInstr& D = hp.dins[j];
    // waits for data the sender already placed (or, skipped, not even that)
    if ((D.op & (OPB_RECV | OPB_LOCAL_IN | OPB_SRCB | OPB_DSTA | OPB_SEND)) == (OPB_RECV | OPB_LOCAL_IN)) continue;
    Range r = op_range(D.pad0, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz);
    // slot reads and writes carry one flag byte per data byte under the LL protocol
    const int slot = (hp.cfg.flags & CCL_FLAG_LL) ? 2 : 1;
    int ops = ((D.op & OPB_RECV) ? slot : 1) + ((D.op & OPB_SRCB) ? 1 : 0) + ((D.op & OPB_DSTA) ? 1 : 0) +
              ((D.op & OPB_SEND) ? slot : 0);
    total += int64_t(ops) * r.len * hp.esz;
  }
  return total;
}

// Exec records of every lowered instruction for `count` elements per rank: byte
// offsets, lengths and slice counts. Slot data starts at the slot's base plus the phase
// of the chunk named by the transfer, so that slot and local operands share their
// 16-byte alignment (LL slots hold units from the base).
void compute_exec_records(const HostPlan& hp, int64_t count, std::vector<DevExec>& out) {
  const int V = 16 / hp.esz;
  const bool ll = hp.cfg.flags & CCL_FLAG_LL;
  out.resize(hp.dins.size());
  auto slot_off = [&](int x) {
    const DevXfer& X = hp.dxf[x];
    if (ll) return int64_t(X.slot_off);
    int64_t ph = 0;
    if (X.phase_idx >= 0) ph = op_range(X.phase_idx, X.cnt, X.instance, hp.k, count, hp.C, 16 / hp.esz).lo % V;
    return int64_t(X.slot_off) + ph * hp.esz;
  };
  for (size_t j = 0; j < hp.dins.size(); ++j) {
    const DevInstr& D = hp.dins[j];
    DevExec E{};
    E.op = D.op | (uint32_t(D.a_buf < 0 ? 0 : D.a_buf) << 8) | (uint32_t(D.b_buf < 0 ? 0 : D.b_buf) << 12) |
           (uint32_t(D.d_buf < 0 ? 0 : D.d_buf) << 16) | ((D.t_buf < 0 ? kStagingBuf : uint32_t(D.t_buf)) << 20) |
           (uint32_t(D.t_rank < 0 ? 0 : D.t_rank) << 24);
    E.xin = D.xin;
    E.xout = D.xout;
    // failure injection: the sender of transfer 0 sets a spare flag (one past the last
    // transfer's) that no receiver waits for, so transfer 0's receiver never sees one
    if ((hp.cfg.flags & CCL_FLAG_DEBUG_DROP_FLAG) && D.xout == 0) E.xout = int32_t(hp.dxf.size());
    E.done_flag = D.done_flag;
    E.wait_begin = D.wait_begin;
    E.nwaits = D.nwaits;
    E.len = op_range(D.pad0, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz).len;
    const int64_t nsl = E.len == 0 ? 0 : (E.len + hp.slice_elems - 1) / hp.slice_elems;
    if (nsl >= (int64_t(1) << kEpochShift)) fail(CCL_ERR_INVALID_ARGUMENT, "too many slices for one transfer");
    E.nsl = int32_t(nsl);
    E.peer_wg = D.peer_wg;
    E.done_peer = D.done_peer;
    if ((D.op & OPB_RECV) && !(D.op & OPB_LOCAL_IN))
      E.a_off = slot_off(D.xin);
    else
      E.a_off = op_range(D.a_idx, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz).lo * hp.esz;
    if (D.op & OPB_SRCB) E.b_off = op_range(D.b_idx, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz).lo * hp.esz;
    if (D.op & OPB_DSTA) E.d_off = op_range(D.d_idx, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz).lo * hp.esz;
    if (D.op & OPB_SEND)
      E.t_off = D.t_buf >= 0 ? op_range(D.t_idx, D.cnt, D.instance, hp.k, count, hp.C, 16 / hp.esz).lo * hp.esz : slot_off(D.xout);
    out[j] = E;
  }
}

// ---------------------------------------------------------------- DAG parallelism

// Parallelism of the instruction DAG (MSCCLang report, section 3.3, which analyses the
// instruction DAG's parallelism): its depth (instructions on the longest dependency
// chain) and width, the largest set of instructions no two of which are ordered (a
// maximum antichain). By Dilworth's theorem the width equals the instruction count
// minus a maximum matching of the bipartite graph that joins u to every v reachable
// from u; the matching is found by Hopcroft-Karp over the transitive closure.
void dag_parallelism(const std::vector<std::set<int>>& succ, int* width, int* depth) {
  const int n = int(succ.size());
  *width = 0;
  *depth = 0;
  if (n == 0) return;
  std::vector<int> key(n);
  std::iota(key.begin(), key.end(), 0);
  const std::vector<int> order = topo_order(succ, key);
  std::vector<int> lvl(n, 1);
  for (int u : order)
    for (int v : succ[u]) lvl[v] = std::max(lvl[v], lvl[u] + 1);
  *depth = *std::max_element(lvl.begin(), lvl.end());
  if (n > 8192) {  // closure would need n^2 bits; report the width as unknown
    *width = -1;
    return;
  }
  const int words = (n + 63) / 64;
  std::vector<uint64_t> reach(size_t(n) * words, 0);
  for (int i = n - 1; i >= 0; --i) {
    const int u = order[i];
    uint64_t* ru = &reach[size_t(u) * words];
    for (int v : succ[u]) {
      ru[v / 64] |= 1ull << (v % 64);
      const uint64_t* rv = &reach[size_t(v) * words];
      for (int w = 0; w < words; ++w) ru[w] |= rv[w];
    }
  }
  std::vector<std::vector<int>> adj(n);
  for (int u = 0; u < n; ++u)
    for (int w = 0; w < words; ++w)
      for (uint64_t b = reach[size_t(u) * words + w]; b; b &= b - 1) adj[u].push_back(w * 64 + __builtin_ctzll(b));
  // Hopcroft-Karp: left copy u -> right copy v for every v reachable from u
  std::vector<int> match_l(n, -1), match_r(n, -1), dist(n);
  auto bfs = [&]() {
    std::queue<int> q;
    bool found = false;
    for (int u = 0; u < n; ++u) {
      dist[u] = match_l[u] < 0 ? 0 : -1;
      if (match_l[u] < 0) q.push(u);
    }
    while (!q.empty()) {
      const int u = q.front();
      q.pop();
      for (int v : adj[u]) {
        const int w = match_r[v];
        if (w < 0) {
          found = true;
        } else if (dist[w] < 0) {
          dist[w] = dist[u] + 1;
          q.push(w);
        }
      }
    }
    return found;
  };
  std::vector<size_t> it(n);
  std::function<bool(int)> dfs = [&](int u) -> bool {
    for (; it[u] < adj[u].size(); ++it[u]) {
      const int v = adj[u][it[u]], w = match_r[v];
      if (w < 0 || (dist[w] == dist[u] + 1 && dfs(w))) {
        match_l[u] = v;
        match_r[v] = u;
        return true;
      }
    }
    dist[u] = -1;
    return false;
  };
  int matching = 0;
  while (bfs()) {
    std::fill(it.begin(), it.end(), 0);
    for (int u = 0; u < n; ++u)
      if (match_l[u] < 0 && dfs(u)) ++matching;
  }
  *width = n - matching;
}

void compile_plan(HostPlan& hp, const ccl_program_desc* prog, int nranks, int nchunks, int k,
                  const ccl_plan_config* cfg) {
  auto t0 = Clock::now();
  validate(hp, prog, nranks, nchunks, k, cfg);
  verify_postcondition(hp);
  hp.ms[0] = ms_since(t0);
  t0 = Clock::now();
  std::vector<std::set<int>> dag;
  fuse(hp, dag);  // DAG construction happens inside; split timing below is approximate
  choose_direct(hp, dag);
  hp.ms[1] = 0.0;
  hp.ms[2] = ms_since(t0);
  t0 = Clock::now();
  schedule(hp, dag);
  dag_parallelism(dag, &hp.dag_width, &hp.dag_depth);
  hp.ms[3] = ms_since(t0);
  t0 = Clock::now();
  allocate_workgroups(hp);
  compute_waits(hp, dag);
  mark_idle_receives(hp, dag);
  hp.ms[4] = ms_since(t0);
  t0 = Clock::now();
  lower(hp);
  hp.ms[5] = ms_since(t0);
}

}  // namespace ccl
