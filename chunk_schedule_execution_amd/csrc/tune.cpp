// AutoCCL-style tuner (AutoCCL report, "Methods" 1 and 2): the implementation choice
// (here: which program, i.e. algorithm) splits the space into subspaces; inside each,
// the resource parameters -- channels/instances (nc), threads per workgroup (nt),
// pipelining chunk (c) -- are tuned one coordinate at a time, each increased while the
// bandwidth keeps improving, relying on its unimodal shape.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <map>
#include <vector>

#include "ccl_internal.h"

using namespace ccl;

namespace {

int index_of(const int32_t* v, int n, int32_t x) {
  for (int i = 0; i < n; ++i)
    if (v[i] == x) return i;
  return 0;
}

// Passes of coordinate descent per subspace at most (each pass visits nc, nt, c once).
constexpr int kMaxPasses = 4;

struct Coord {
  const int32_t* vals;
  int n;
  int32_t ccl_tune_point::*field;
};

}  // namespace

extern "C" {

int ccl_tune_coordinate_descent(const ccl_tune_space* space, const ccl_tune_point* start, ccl_tune_objective objective,
                                void* user, ccl_tune_point* best, ccl_tune_report* report) {
  if (!space || !objective || !best || !report) return CCL_ERR_INVALID_ARGUMENT;
  if (space->nfactors < 1 || space->nnthreads < 1 || space->nslices < 1 || space->nvariants < 1 || !space->factors ||
      !space->nthreads || !space->slices)
    return CCL_ERR_INVALID_ARGUMENT;
  const Coord coords[3] = {{space->factors, space->nfactors, &ccl_tune_point::parallel_factor},
                           {space->nthreads, space->nnthreads, &ccl_tune_point::nthreads},
                           {space->slices, space->nslices, &ccl_tune_point::slice_bytes}};
  int evals = 0;
  bool have_best = false;
  double best_score = -1.0, start_score = -1.0;
  const int protos = space->protocols ? space->protocols : 1;
  bool first = true;
  for (int v = 0; v < space->nvariants; ++v) {
    for (int proto = 0; proto < 4; ++proto) {
      if (!(protos & (1 << proto))) continue;
      ccl_tune_point pt{};
      pt.variant = v;
      pt.protocol = proto;
      // objective values of this subspace by candidate indices: a point is timed once
      std::map<std::array<int, 3>, double> seen;
      auto eval = [&](const int* ix) {
        const std::array<int, 3> key{ix[0], ix[1], ix[2]};
        auto it = seen.find(key);
        if (it != seen.end()) return it->second;
        ccl_tune_point q = pt;
        for (int c = 0; c < 3; ++c) q.*(coords[c].field) = coords[c].vals[ix[c]];
        const double score = objective(&q, user);
        ++evals;
        seen.emplace(key, score);
        return score;
      };
      // One coordinate descent from `from`; returns its score and leaves its point in `at`.
      // Each coordinate moves in direction dir (+1 / -1) while the objective improves,
      // looking one candidate past a step that does not improve (resource counts that
      // leave part of the machine idle can dip between two better values). The first pass
      // raises each coordinate from its start (and, from a start inside the space, lowers
      // it if raising does not help); later passes (repeated until a whole pass changes
      // nothing) move each coordinate up or, failing that, down from where the others now
      // are: the best thread count can depend on the slice size chosen after it.
      auto descend = [&](const int* from, bool inside, int* at) {
        int idx[3] = {from[0], from[1], from[2]};
        double score = eval(idx);
        auto climb = [&](int c, int dir) {
          bool moved = false;
          for (;;) {
            int ix[3] = {idx[0], idx[1], idx[2]};
            ix[c] = idx[c] + dir;
            if (ix[c] < 0 || ix[c] >= coords[c].n) break;
            double s = eval(ix);
            if (!(s > score)) {
              ix[c] += dir;
              if (ix[c] < 0 || ix[c] >= coords[c].n) break;
              s = eval(ix);
              if (!(s > score)) break;
            }
            idx[c] = ix[c];
            score = s;
            moved = true;
          }
          return moved;
        };
        for (int pass = 0; pass < kMaxPasses; ++pass) {
          bool changed = false;
          for (int c = 0; c < 3; ++c) {
            bool m = climb(c, +1);
            if (!m && (pass > 0 || inside)) m = climb(c, -1);
            changed |= m;
          }
          if (!changed) break;
        }
        for (int c = 0; c < 3; ++c) at[c] = idx[c];
        return score;
      };
      // Two descents per subspace, from the given start (else the space's corner) and
      // from the middle of every coordinate; the better end point counts. A descent from
      // the corner alone stopped at local peaks: a 16-rank bf16 hierarchical AllReduce at
      // 128 MiB ended at a point slower than the three-launch composition it replaces.
      int from0[3], mid[3], idx[3], idx2[3];
      for (int c = 0; c < 3; ++c) {
        from0[c] = start ? index_of(coords[c].vals, coords[c].n, start->*(coords[c].field)) : 0;
        mid[c] = coords[c].n / 2;
      }
      if (first) start_score = eval(from0);
      first = false;
      double score = descend(from0, false, idx);
      const double score2 = descend(mid, true, idx2);
      if (score2 > score) {
        score = score2;
        for (int c = 0; c < 3; ++c) idx[c] = idx2[c];
      }
      for (int c = 0; c < 3; ++c) pt.*(coords[c].field) = coords[c].vals[idx[c]];
      if (score >= 0 && (!have_best || score > best_score)) {
        have_best = true;
        best_score = score;
        *best = pt;
      }
    }
  }
  report->evaluations = evals;
  report->best_score = best_score;
  report->start_score = start_score;
  return have_best ? CCL_OK : CCL_ERR_OUT_OF_RESOURCES;
}

struct DeviceTuneCtx {
  const ccl_program_desc* const* variants;
  int64_t count;
  ccl_plan_config base;
  hipStream_t stream;
  int warmup, iters;
  std::vector<void*> in, out;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int last_error;
};

static double device_objective(const ccl_tune_point* pt, void* user) {
  auto* c = static_cast<DeviceTuneCtx*>(user);
  const ccl_program_desc* prog = c->variants[pt->variant];
  ccl_plan_config cfg = c->base;
  cfg.nthreads = pt->nthreads;
  cfg.slice_bytes = pt->slice_bytes;
  cfg.flags &= ~(CCL_FLAG_HOST_ONLY | CCL_FLAG_TRACE | CCL_FLAG_LL | CCL_FLAG_DIRECT | CCL_FLAG_STREAMING);
  if (pt->protocol == 1) cfg.flags |= CCL_FLAG_LL;
  if (pt->protocol >= 2) cfg.flags |= CCL_FLAG_DIRECT;
  if (pt->protocol == 3) cfg.flags |= CCL_FLAG_STREAMING;
  ccl_plan* plan = nullptr;
  int rc = ccl_plan_create(prog, prog->nranks, prog->in_chunks, pt->parallel_factor, &cfg, &plan);
  if (rc) return -1.0;  // infeasible (e.g. not enough co-resident workgroups)
  for (int i = 0; i < c->warmup && rc == 0; ++i)
    rc = ccl_execute(plan, (const void* const*)c->in.data(), c->out.data(), c->count, c->stream);
  (void)hipEventRecord(c->e0, c->stream);
  for (int i = 0; i < c->iters && rc == 0; ++i)
    rc = ccl_execute(plan, (const void* const*)c->in.data(), c->out.data(), c->count, c->stream);
  (void)hipEventRecord(c->e1, c->stream);
  (void)hipEventSynchronize(c->e1);
  if (rc == 0) rc = ccl_plan_status(plan);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, c->e0, c->e1);
  ccl_plan_destroy(plan);
  if (rc) {
    c->last_error = rc;
    return -1.0;
  }
  double t = ms * 1e-3 / std::max(1, c->iters);
  int esz = c->base.dtype == CCL_BF16 ? 2 : 4;
  return t > 0 ? double(c->count) * esz / t / 1e9 : -1.0;  // algorithm bandwidth, GB/s
}

int ccl_tune(const ccl_program_desc* const* variants, int nvariants, int64_t count, const ccl_plan_config* base,
             const ccl_tune_space* space, void* stream, ccl_tune_point* best, ccl_tune_report* report) {
  if (!variants || nvariants < 1 || !base || !space || !best || !report || count < 1) return CCL_ERR_INVALID_ARGUMENT;
  int P = variants[0]->nranks;
  for (int v = 0; v < nvariants; ++v)
    if (!variants[v] || variants[v]->nranks != P || variants[v]->collective != variants[0]->collective)
      return CCL_ERR_INVALID_ARGUMENT;
  DeviceTuneCtx c;
  c.variants = variants;
  c.count = count;
  c.base = *base;
  c.base.max_count = std::max<int64_t>(base->max_count, count);
  c.stream = reinterpret_cast<hipStream_t>(stream);
  c.warmup = std::max(0, space->warmup);
  c.iters = std::max(1, space->iters);
  c.last_error = 0;
  int esz = base->dtype == CCL_BF16 ? 2 : 4;
  // buffer sizes: the largest output any supported collective needs for count
  ccl_program_desc probe = *variants[0];
  int64_t oc = output_chunks(probe);
  int64_t out_elems = oc >= 0 ? (oc * count) / probe.in_chunks + 1 : count * P;
  int rc = CCL_OK;
  for (int r = 0; r < P && rc == 0; ++r) {
    void* a = nullptr;
    void* b = nullptr;
    if (hipMalloc(&a, size_t(count) * esz) != hipSuccess || hipMalloc(&b, size_t(out_elems) * esz) != hipSuccess) {
      if (a) (void)hipFree(a);
      rc = CCL_ERR_OUT_OF_RESOURCES;
      break;
    }
    (void)hipMemset(a, 0, size_t(count) * esz);
    c.in.push_back(a);
    c.out.push_back(b);
  }
  if (rc == 0 && (hipEventCreate(&c.e0) != hipSuccess || hipEventCreate(&c.e1) != hipSuccess)) rc = CCL_ERR_HIP;
  ccl_tune_space sp = *space;
  sp.nvariants = nvariants;
  if (rc == 0) rc = ccl_tune_coordinate_descent(&sp, nullptr, device_objective, &c, best, report);
  (void)hipDeviceSynchronize();
  for (void* p : c.in) (void)hipFree(p);
  for (void* p : c.out) (void)hipFree(p);
  if (c.e0) (void)hipEventDestroy(c.e0);
  if (c.e1) (void)hipEventDestroy(c.e1);
  return rc;
}

}  // extern "C"
