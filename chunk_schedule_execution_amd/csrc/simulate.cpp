// Host-side check of a lowered plan (no GPU, no floating point).
//
// Runs every workgroup's lowered instruction list under the executor's flag
// protocol -- a receiver's slice s may run once the sender has finished slice s, an
// instruction with completion waits starts once those instructions are done -- in
// seeded random interleavings, one slice at a time. Values are multisets of
// contributing input elements (rank, element), so the outcome is compared with the
// collective's postcondition symbolically. A state where no workgroup can move but
// some are unfinished is a deadlock; a read of a scratch element never written is an
// ordering bug. This checks the compiler's output (fusion, scheduling, workgroup
// merging, waits); it is not a way of computing a collective.
#include <algorithm>
#include <cstdio>

#include "ccl_internal.h"

namespace ccl {

namespace {

struct Val {
  bool init = false;
  std::vector<uint32_t> atoms;  // sorted
};

constexpr uint32_t kPriorAtom = 0x80000000u;

inline uint32_t atom(int r, int64_t e) { return uint32_t(r) << 20 | uint32_t(e); }

struct Rng {
  uint64_t s;
  uint64_t next() {  // splitmix64
    uint64_t z = (s += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
  }
};

}  // namespace

void check_lowered(const HostPlan& hp, uint64_t seed, int nsims) {
  const int P = hp.P;
  // element count: a multiple of the count granule with about three elements per instance sub-chunk
  int64_t min_count = int64_t(3) * hp.C * hp.k;
  int64_t N = ((min_count + hp.granule - 1) / hp.granule) * hp.granule;
  if (N >= (int64_t(1) << 20)) fail(CCL_ERR_INVALID_ARGUMENT, "plan too large for the host check");
  const int64_t se = 2;  // slice length in the simulation: several slices per instruction
  const int64_t nout = output_elems(hp, N);
  const int64_t nscr = chunk_bound(hp.scr_chunks, N, hp.C);
  const int nW = int(hp.dwg.size());
  const int nX = int(hp.dxf.size());
  int nD = 0;
  for (const auto& D : hp.dins) nD = std::max(nD, D.done_flag + 1);

  for (int sim = 0; sim < nsims; ++sim) {
    Rng rng{seed * 0x100000001b3ULL + uint64_t(sim) + 1};
    std::vector<std::vector<Val>> buf[3];
    for (int b = 0; b < 3; ++b) buf[b].resize(P);
    for (int r = 0; r < P; ++r) {
      buf[0][r].resize(N);
      for (int64_t e = 0; e < N; ++e) buf[0][r][e] = {true, {atom(r, e)}};
      buf[1][r].resize(nout);
      for (int64_t e = 0; e < nout; ++e) buf[1][r][e] = {true, {kPriorAtom | atom(r, e)}};
      buf[2][r].assign(nscr, Val{});
    }
    std::vector<std::vector<Val>> slot(nX);
    std::vector<int64_t> xflag(nX, 0);
    std::vector<char> dflag(nD, 0);
    std::vector<int> ip(nW, 0);
    std::vector<int64_t> sl(nW, 0);
    std::vector<char> started(nW, 0);
    // Lazy loop order (CCL_FLAG_LAZY): iteration it runs slice it of every instruction of
    // the workgroup in order; an instruction with e = max(slices, 1) takes part in
    // iterations 0 .. e-1, its completion waits at 0 and its completion flag at e-1.
    // (an LL instruction is one pass either way, so LL plans run in task order)
    const bool lazy = (hp.cfg.flags & CCL_FLAG_LAZY) && !(hp.cfg.flags & CCL_FLAG_LL);
    std::vector<int64_t> iters(nW, 1), lit(nW, 0);
    // instruction geometry at N
    struct Geo {
      int64_t len, alo, blo, dlo, tlo, nsl;
    };
    std::vector<Geo> geo(hp.dins.size());
    for (size_t j = 0; j < hp.dins.size(); ++j) {
      const DevInstr& D = hp.dins[j];
      Geo g{};
      g.len = op_range(D.pad0, D.cnt, D.instance, hp.k, N, hp.C, 16 / hp.esz).len;
      const bool local_a = !(D.op & OPB_RECV) || (D.op & OPB_LOCAL_IN);
      if (local_a) g.alo = op_range(D.a_idx, D.cnt, D.instance, hp.k, N, hp.C, 16 / hp.esz).lo;
      if (D.t_buf >= 0) g.tlo = op_range(D.t_idx, D.cnt, D.instance, hp.k, N, hp.C, 16 / hp.esz).lo;
      if (D.op & OPB_SRCB) g.blo = op_range(D.b_idx, D.cnt, D.instance, hp.k, N, hp.C, 16 / hp.esz).lo;
      if (D.op & OPB_DSTA) g.dlo = op_range(D.d_idx, D.cnt, D.instance, hp.k, N, hp.C, 16 / hp.esz).lo;
      g.nsl = (g.len + se - 1) / se;
      geo[j] = g;
      if ((D.op & OPB_SEND) && D.t_buf < 0) slot[D.xout].assign(g.len, Val{});
    }
    auto eff = [&](int j) { return std::max<int64_t>(1, geo[j].nsl); };
    if (lazy) {
      for (int w = 0; w < nW; ++w)
        for (int t = 0; t < hp.dwg[w].n; ++t) iters[w] = std::max(iters[w], eff(hp.dwg[w].first + t));
    }
    // lazy: skip instructions that take no part in the current iteration
    auto lazy_settle = [&](int w) {
      const DevWG& G = hp.dwg[w];
      for (;;) {
        if (lit[w] >= iters[w]) return;
        if (ip[w] >= G.n) {
          ip[w] = 0;
          ++lit[w];
          continue;
        }
        if (lit[w] < eff(G.first + ip[w])) return;
        ++ip[w];
      }
    };
    if (lazy)
      for (int w = 0; w < nW; ++w) lazy_settle(w);
    std::vector<int> runnable;
    for (;;) {
      runnable.clear();
      bool all_done = true;
      for (int w = 0; w < nW; ++w) {
        const DevWG& G = hp.dwg[w];
        if (lazy ? lit[w] >= iters[w] || G.n == 0 : ip[w] >= G.n) continue;
        all_done = false;
        int j = G.first + ip[w];
        const DevInstr& D = hp.dins[j];
        const int64_t s_now = lazy ? lit[w] : sl[w];
        if (lazy ? s_now == 0 : !started[w]) {
          bool ok = true;
          for (int q = 0; q < D.nwaits; ++q)
            if (!dflag[hp.dwaits[D.wait_begin + q]]) ok = false;
          if (!ok) continue;
        }
        if ((D.op & OPB_RECV) && !(D.op & OPB_SKIP) && s_now < geo[j].nsl && xflag[D.xin] < s_now + 1) continue;
        runnable.push_back(w);
      }
      if (all_done) break;
      if (runnable.empty()) {
        char msg[160];
        snprintf(msg, sizeof msg, "deadlock in interleaving %d: no workgroup can proceed", sim);
        fail(CCL_ERR_INVALID_PROGRAM, msg);
      }
      int w = runnable[rng.next() % runnable.size()];
      const DevWG& G = hp.dwg[w];
      int j = G.first + ip[w];
      const DevInstr& D = hp.dins[j];
      const Geo& g = geo[j];
      started[w] = 1;
      if (lazy) sl[w] = lit[w];
      if (D.op & OPB_SKIP) {
        // a skipped receive has run its completion waits (checked above) and then
        // waits for no transfer flag and touches nothing
        if (lazy) {
          ip[w]++;
          lazy_settle(w);
        } else {
          ip[w]++;
          sl[w] = 0;
          started[w] = 0;
        }
        continue;
      }
      if (sl[w] < g.nsl) {
        int64_t lo = sl[w] * se, hi = std::min(g.len, lo + se);
        for (int64_t e = lo; e < hi; ++e) {
          const bool from_slot = (D.op & OPB_RECV) && !(D.op & OPB_LOCAL_IN);
          Val v = from_slot ? slot[D.xin][e] : buf[D.a_buf][G.rank][g.alo + e];
          if (D.op & OPB_SRCB) {
            const Val& b = buf[D.b_buf][G.rank][g.blo + e];
            if (!b.init) v.init = false;
            std::vector<uint32_t> m;
            std::merge(v.atoms.begin(), v.atoms.end(), b.atoms.begin(), b.atoms.end(), std::back_inserter(m));
            v.atoms.swap(m);
          }
          if (!v.init) {
            char msg[200];
            snprintf(msg, sizeof msg, "instruction %d of workgroup %d reads an element that was never written", ip[w], w);
            fail(CCL_ERR_INVALID_PROGRAM, msg);
          }
          if (D.op & OPB_DSTA) buf[D.d_buf][G.rank][g.dlo + e] = v;
          if ((D.op & OPB_SEND) && D.t_buf >= 0)
            buf[D.t_buf][D.t_rank][g.tlo + e] = v;  // direct transport: the receiver's own location
          else if (D.op & OPB_SEND)
            slot[D.xout][e] = v;
        }
        if ((D.op & OPB_SEND) && !(D.op & OPB_NOFLAG)) xflag[D.xout] = sl[w] + 1;
        sl[w]++;
      }
      if (lazy) {
        if (lit[w] == eff(j) - 1 && D.done_flag >= 0) dflag[D.done_flag] = 1;
        ip[w]++;
        lazy_settle(w);
      } else if (sl[w] >= g.nsl) {
        if (D.done_flag >= 0) dflag[D.done_flag] = 1;
        ip[w]++;
        sl[w] = 0;
        started[w] = 0;
      }
    }
    // postcondition
    const ccl_program_desc& d = hp.desc;
    if (d.collective == CCL_COLL_CUSTOM) continue;
    int n = group_count(d);
    std::vector<int> M;
    for (int r = 0; r < P; ++r) {
      int p;
      group_members(d, r, M, p);
      for (int64_t e = 0; e < nout; ++e) {
        std::vector<uint32_t> want;
        switch (d.collective) {
          case CCL_COLL_ALLREDUCE:
            for (int m : M) want.push_back(atom(m, e));
            break;
          case CCL_COLL_ALLGATHER:
            want.push_back(atom(M[e / N], e % N));
            break;
          case CCL_COLL_REDUCESCATTER: {
            int64_t sh = N / n;
            for (int m : M) want.push_back(atom(m, p * sh + e));
            break;
          }
          case CCL_COLL_ALLTOALL: {
            int64_t b = N / n;
            want.push_back(atom(M[e / b], p * b + e % b));
            break;
          }
          case CCL_COLL_ALLTONEXT:
            want.push_back(p == 0 ? (kPriorAtom | atom(r, e)) : atom(M[p - 1], e));
            break;
        }
        std::sort(want.begin(), want.end());
        if (buf[1][r][e].atoms != want) {
          char msg[200];
          snprintf(msg, sizeof msg, "interleaving %d: rank %d output element %lld violates the postcondition", sim, r,
                   (long long)e);
          fail(CCL_ERR_INVALID_PROGRAM, msg);
        }
      }
    }
  }
}

}  // namespace ccl
