/*
 * ccl.h -- C ABI of the chunk-schedule collective executor for MI355X (gfx950).
 *
 * A collective is written as a chunk program: copy and reduce operations on
 * chunks of per-rank input, output and scratch buffers, in program order
 * (MSCCLang report, section 3.1 "System design": the chunk-oriented DSL, its
 * input/output/scratch buffers and copy/reduce operations). ccl_plan_create
 * compiles it once: dependency DAG, send/recv instruction generation, fusion into
 * recv-reduce-copy-send style instructions, replication into parallel instances
 * on separate channels (MSCCLang report, section 3.1, compiler steps), scheduling
 * into sub-pipelines with hierarchical-priority dynamic scheduling and merging of
 * never co-active connections onto one workgroup (ReSCCL report, section 2.2
 * "System design"). ccl_execute then runs the whole collective as one HIP kernel
 * launch on a stream.
 *
 * The P ranks are virtual ranks that live on one GPU: every rank's buffers sit
 * in the same HBM, a "send" writes the receiving rank's staging slot and then
 * release-stores a flag, a "recv" acquire-polls that flag and reads the slot.
 *
 * The stream of a plan's last launch must stay valid until the next execute, status or
 * destroy call on that plan.
 *
 * Conventions for every entry point:
 *   - Status codes: CCL_OK (0) on success, a negative CCL_ERR_* otherwise. No C++
 *     exception crosses this boundary. ccl_last_error_detail() gives a
 *     thread-local text for the last failure of the calling thread.
 *   - Pointers named "device" are HIP device pointers owned by the caller. All
 *     other pointers are host pointers owned by the caller and only read during
 *     the call unless stated otherwise.
 *   - A stream argument is a hipStream_t passed as void* (NULL = null stream).
 *   - Element counts are in elements of the plan's dtype; chunk indices and chunk
 *     counts are in chunks.
 */
#ifndef CCL_H
#define CCL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define CCL_OK 0
#define CCL_ERR_INVALID_ARGUMENT (-1) /* bad sizes, pointers, counts, or mismatched parameters */
#define CCL_ERR_INVALID_PROGRAM (-2)  /* program fails verification (bounds, input writes, postcondition, ...) */
#define CCL_ERR_UNSUPPORTED (-3)      /* dtype / reduction / collective not supported */
#define CCL_ERR_OUT_OF_RESOURCES (-4) /* more workgroups than can be co-resident, or allocation failure */
#define CCL_ERR_HIP (-5)              /* a HIP runtime call failed */
#define CCL_ERR_TIMEOUT (-6)          /* a device spin-wait exceeded its watchdog budget */
#define CCL_ERR_INTERNAL (-7)

/* ---- program description (MSCCLang report, section 3.1: chunks, buffers, copy/reduce) ---- */
#define CCL_OP_COPY 0   /* dst <- src */
#define CCL_OP_REDUCE 1 /* dst <- dst + src (one storage-dtype rounding) */

#define CCL_BUF_INPUT 0   /* read-only per-rank input (the caller's send buffer) */
#define CCL_BUF_OUTPUT 1  /* per-rank output (the caller's receive buffer) */
#define CCL_BUF_SCRATCH 2 /* per-rank scratch owned by the plan */

#define CCL_REDOP_SUM 0

#define CCL_F32 0
#define CCL_BF16 1 /* stored as bf16, added in fp32, rounded to nearest-even at every store */
#define CCL_I32 2  /* two's-complement wrap */

/* Collective: picks the postcondition the verifier checks and the buffer sizes. */
#define CCL_COLL_ALLREDUCE 0     /* out = N elements */
#define CCL_COLL_ALLGATHER 1     /* out = P*N (or L*N with CCL_SCOPE_INTRA) */
#define CCL_COLL_REDUCESCATTER 2 /* out = N/P (or N/L with CCL_SCOPE_INTRA); N must divide */
#define CCL_COLL_ALLTOALL 3      /* out = N */
#define CCL_COLL_ALLTONEXT 4     /* out = N; rank 0's output is left untouched */
#define CCL_COLL_CUSTOM 5        /* no postcondition check; out_chunks taken from the program */

/* Group scope for P = G*L ranks numbered r = g*L + l. */
#define CCL_SCOPE_ALL 0   /* the collective spans all P ranks */
#define CCL_SCOPE_INTRA 1 /* an independent collective inside each group of L consecutive ranks */
#define CCL_SCOPE_INTER 2 /* an independent collective among the G ranks of each lane l */

typedef struct {
  uint8_t kind;     /* CCL_OP_COPY or CCL_OP_REDUCE */
  uint8_t redop;    /* CCL_REDOP_SUM */
  uint16_t channel; /* channel label; instructions of different channels never share a workgroup
                       under connection-based allocation */
  int32_t src_rank, src_buf, src_idx;
  int32_t dst_rank, dst_buf, dst_idx;
  int32_t count; /* chunks covered, >= 1 */
} ccl_chunk_op;  /* 32 bytes */

typedef struct {
  int32_t collective;     /* CCL_COLL_* */
  int32_t nranks;         /* P */
  int32_t in_chunks;      /* chunks the input of N elements is cut into (the plan's chunk unit) */
  int32_t out_chunks;     /* chunks of the output buffer */
  int32_t scratch_chunks; /* chunks of per-rank scratch (0 if unused) */
  int32_t group_size;     /* L for CCL_SCOPE_INTRA / CCL_SCOPE_INTER, else ignored */
  int32_t group_scope;    /* CCL_SCOPE_* */
  int32_t reserved;
  const ccl_chunk_op* ops; /* host array of nops operations, in program order; copied by create */
  size_t nops;
} ccl_program_desc;

/*
 * Chunk geometry. With N = count elements per rank input and C = in_chunks, chunk
 * j of every buffer covers elements [floor(j*N/C), floor((j+1)*N/C)); buffers longer
 * than the input simply have more chunks. With parallel factor k > 1 each chunk
 * is split the same way into k instance sub-chunks and instance i runs on its own
 * channel (MSCCLang report, section 3.1: parallelization factor and channels).
 */

/* ---- plan configuration -------------------------------------------------- */
#define CCL_SCHED_PROGRAM_ORDER 0 /* every workgroup runs its tasks in program order */
#define CCL_SCHED_HPDS 1          /* hierarchical-priority dynamic scheduling (ReSCCL report, section 2.2) */
#define CCL_SCHED_RR 2            /* round-robin over chunks, no link-conflict check */

#define CCL_WG_CONNECTION 0 /* one workgroup per (channel, recv peer, send peer) signature of a rank */
#define CCL_WG_STATE 1      /* additionally merge workgroups of one rank that are never co-active */

#define CCL_FLAG_TRACE 0x1u      /* record per-workgroup busy/wait timestamps (ccl_plan_read_trace) */
#define CCL_FLAG_HOST_ONLY 0x2u  /* compile and lower on the host only; no HIP call, no execute */
#define CCL_FLAG_NO_FUSION 0x4u  /* keep primitive send/recv/copy/reduce instructions */
#define CCL_FLAG_NO_VERIFY 0x8u  /* skip the symbolic postcondition check at create */
#define CCL_FLAG_LL 0x10u        /* low-latency protocol: every 4 data bytes in a staging slot travel with a
                                    4-byte flag in one 8-byte store; receivers poll the data itself, there
                                    are no per-slice flags (twice the slot traffic, far fewer round trips;
                                    the protocol choice of the MSCCLang report, section 3.1 runtime, and the
                                    AutoCCL report's Protocol parameter) */
#define CCL_FLAG_DIRECT 0x40u     /* direct transport (simple protocol only): the sender writes a transfer
                                    into the receiving rank's own memory instead of a staging slot. A
                                    receive that copies the data into a local location has it written there
                                    and only waits for the transfer's flag (forwarding from its own buffer);
                                    a reducing receive that only forwards its sum has it written into the
                                    same chunk of the receiver's output (else scratch) buffer and adds its
                                    local operand there. Applied to a transfer when every other instruction
                                    of the receiving rank that touches that location runs after the receive
                                    or before the sender. The AutoCCL report's transport parameter; ring
                                    AllReduce moves S(5P-4) bytes instead of S(6P-4), with no slots */
#define CCL_FLAG_STREAMING 0x80u  /* non-temporal hint on local-buffer loads and stores (simple protocol):
                                    streamed lines are not kept in the caches. Helps when the working set is
                                    far larger than the caches, costs when it fits */
#define CCL_FLAG_FORCE_XCD_LOCAL 0x100u /* use the XCD-local variant even when the layout spreads transfers over
                                    XCDs: senders then find most receivers on other XCDs and release each
                                    flag. Slow; exists to exercise that path */
#define CCL_FLAG_SPECIALIZE 0x200u /* run a kernel generated for this plan instead of the interpreting one
                                    (ReSCCL report, section 2.2, lightweight kernel generation), compiled with
                                    hiprtc at create (code objects cached per process). When the plan's
                                    distinct workgroup programs hold at most 24 instructions in all, each
                                    becomes straight-line code with the operations and buffers as constants;
                                    longer plans get the loop form (CCL_FLAG_SPECIALIZE_LOOP), whose code stays
                                    within the instruction cache. Same records, flags and results; with
                                    HOST_ONLY the kernel is generated and compiled but not loaded. Compile
                                    failures give CCL_ERR_HIP */
#define CCL_FLAG_SPECIALIZE_LOOP 0x800u /* a generated kernel in the loop form: each workgroup walks its
                                    records and switches over the plan's distinct operation words, one step
                                    with constant operation and buffers per word */
#define CCL_FLAG_LAZY 0x400u      /* with or without SPECIALIZE: a generated kernel that runs the lazy loop
                                    order, slice s of every instruction of a workgroup before slice s + 1 of
                                    any (the algorithm once per slice; ReSCCL report, section 2.1), instead of
                                    every slice of an instruction before the next. CCL_ERR_UNSUPPORTED for
                                    plans with cross-workgroup completion waits */
#define CCL_FLAG_DEBUG_DROP_FLAG 0x1000u /* failure injection for tests of the watchdog (simple protocol): the
                                    sender of transfer 0 never sets its flag, so its receiver waits out the
                                    watchdog budget (timeout_us) and every launch of the plan ends with
                                    CCL_ERR_TIMEOUT from ccl_plan_status; every workgroup still leaves.
                                    Refused (CCL_ERR_UNSUPPORTED) with CCL_FLAG_LL, whose flags travel inside
                                    the data, and with CCL_FLAG_DIRECT, where a receive that ends its
                                    workgroup is not waited for */
#define CCL_FLAG_DEBUG_POISON 0x2000u /* debug mode: before every launch, on the launch's stream, fill the plan's
                                    staging slots and scratch with the byte 0xFA (fp32 -6.5e35, bf16 -6.5e35,
                                    int32 -84215046; as a low-latency unit its flag word is never a launch's),
                                    so that a read of a slot or scratch location before its producer wrote
                                    it in this launch shows up in the outputs. Results are unchanged
                                    otherwise; costs one fill per launch */
#define CCL_FLAG_COHERENT_ONLY 0x20u /* write transfers and their flags with agent-coherent stores. By default a
                                    plan whose lowered layout keeps every transfer on one XCD (workgroup ids
                                    congruent mod 8, which the round-robin dispatch places together) writes
                                    transfer data with plain stores; each sender then checks the XCD its
                                    receiving workgroup published at the start of the launch and, when it is
                                    its own, sets the flag with a plain store (data and flag meet in that
                                    XCD's shared L2); otherwise the flag store is a full agent-scope release */

typedef struct {
  int32_t dtype;       /* CCL_F32, CCL_BF16 or CCL_I32 */
  int32_t redop;       /* CCL_REDOP_SUM */
  int64_t max_count;   /* largest per-rank input element count ccl_execute will be given (>= 1) */
  int32_t nthreads;    /* threads per workgroup: 64..1024, multiple of 64 (0 = 512) */
  int32_t slice_bytes; /* pipelining slice per transfer step, bytes (0 = 256 KiB) */
  int32_t scheduler;   /* CCL_SCHED_* */
  int32_t wg_alloc;    /* CCL_WG_* */
  uint32_t flags;      /* CCL_FLAG_* */
  int32_t num_cus;     /* compute-unit budget (0 = the whole device). The co-residency check bounds the
                          grid by occupancy x min(num_cus, the device's CUs), so a plan sized for a budget
                          leaves the other CUs to concurrent work (AutoCCL report, method 3: tuning while
                          computation holds part of the GPU; ReSCCL report, section 1: thread blocks taken
                          from computation). HOST_ONLY plans assume num_cus CUs (0 = 256). The layout keeps
                          every instance on one XCD only when the padded grid fits num_cus (0 = 256) */
  int64_t timeout_us;  /* watchdog budget of one device spin-wait, microseconds (0 = 2,000,000) */
} ccl_plan_config;

typedef struct ccl_plan ccl_plan;

/*
 * Compile `prog` into a plan. `nranks` must equal prog->nranks and `nchunks`
 * prog->in_chunks (both are restated so that a caller cannot pair a program with
 * the wrong shape silently). `parallel_factor` k >= 1 replicates the program into
 * k instances. Unless CCL_FLAG_HOST_ONLY is set the plan allocates its device
 * memory (instruction tables, staging slots sized for max_count, flags, scratch)
 * on the current HIP device and checks that every workgroup can be resident at
 * once. The plan is immutable afterwards.
 * Errors: INVALID_ARGUMENT (sizes, mismatched nranks/nchunks, null pointers),
 * INVALID_PROGRAM (chunk out of range, write to an input, length mismatch, failed
 * postcondition), UNSUPPORTED, OUT_OF_RESOURCES (too many workgroups,
 * hipMalloc failure), HIP. On error *out is NULL and nothing is leaked.
 */
int ccl_plan_create(const ccl_program_desc* prog, int nranks, int nchunks, int parallel_factor,
                    const ccl_plan_config* cfg, ccl_plan** out);

/*
 * Run the collective once on `stream`: sendbufs[r] / recvbufs[r] (r < P) are
 * device pointers to rank r's input (count elements) and output (the
 * collective's output length for count). Out of place: outputs must not overlap
 * inputs. Enqueues exactly one kernel (none when count == 0) and returns at once;
 * the buffers must stay valid until the stream passes the kernel. Launches of one
 * plan are serialized: a launch on another stream first waits for the previous one.
 * Errors: INVALID_ARGUMENT (count > max_count, count not a multiple of the plan's
 * count granule or of P where the collective needs it, null pointers, HOST_ONLY
 * plan), UNSUPPORTED when `stream` is capturing a graph (every launch carries a fresh
 * epoch, which a graph replay would repeat), HIP. A watchdog expiry during a launch is
 * reported by ccl_plan_status.
 */
int ccl_execute(ccl_plan* plan, const void* const* sendbufs, void* const* recvbufs, int64_t count,
                void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture set-up,
 * tight serving loops, harnesses that forbid hipMalloc. Runs the collective of `plan`
 * like ccl_execute (same arguments, same results bit for bit) but allocates nothing:
 * no hipMalloc, hipFree or allocating library call. `plan` may be a CCL_FLAG_HOST_ONLY
 * plan, which owns no device memory at all; a device plan's own memory is not used.
 * Every device-side word of the launch -- transfer and completion flags, workgroup XCD
 * tags, the error word, the workgroup table, the instruction records, staging slots
 * and scratch -- lives in the library's static device scratch, one 64 MiB array per GPU,
 * held from the first such call on that GPU until the process ends. The interpreting
 * kernel runs (a plan's generated kernel is not loaded; trace recording is off).
 * Per GPU the array keeps the last call's contents: tables are uploaded only when the
 * plan or count differs from that call (a synchronous copy on `stream`), launch epochs
 * rise across all calls on the GPU so flags left by earlier calls never satisfy a wait,
 * and the error word (plus, for CCL_FLAG_LL, the slots) is cleared on `stream` before
 * the launch. Calls on one GPU share the array: calls that overlap in time (on
 * different streams, or from several threads) race and give undefined results; keep
 * them on one stream. ccl_plan_status(plan) reports a watchdog expiry of the plan's
 * last call here (the error word is shared, so only until the next call on that GPU).
 * Errors: as ccl_execute, and OUT_OF_RESOURCES when the plan needs more than the array
 * holds (64 MiB in all, of which 57.7 MiB for tables, records, slots and scratch;
 * 32,768 transfer flags, 16,384 completion flags, 8,192 workgroups) or more co-resident
 * workgroups of the interpreting kernel than the device (or the plan's CU budget) holds.
 */
int ccl_execute_static(ccl_plan* plan, const void* const* sendbufs, void* const* recvbufs, int64_t count,
                       void* stream);

/* Wait for the plan's last launch and free everything it owns. NULL is a no-op. */
int ccl_plan_destroy(ccl_plan* plan);

typedef struct {
  int32_t nranks, nchunks, parallel_factor, dtype;
  int32_t num_workgroups;     /* workgroups that run instructions, all ranks and instances */
  int32_t max_wg_per_rank;
  int32_t num_instructions;   /* lowered, all instances */
  int32_t num_subpipelines;   /* of the base schedule */
  int32_t num_connections;    /* distinct (src rank, dst rank, channel), all instances */
  int32_t num_transfers;      /* send->recv pairs, all instances */
  int32_t num_waits;          /* cross-workgroup completion waits, all instances */
  int32_t count_granule;      /* ccl_execute's count must be a multiple of this */
  int32_t nthreads, slice_bytes;
  int32_t max_resident_wgs;   /* co-residency bound the plan was checked against */
  int32_t grid_workgroups;    /* launch grid: num_workgroups plus idle ids that keep every instance on one XCD */
  int32_t xcd_local;          /* 1: XCD-local layout, plain transfer stores (see CCL_FLAG_COHERENT_ONLY) */
  int32_t specialized_shapes; /* generated kernel (CCL_FLAG_SPECIALIZE / LAZY): distinct instruction
                                 sequences in it; 0 for the interpreting kernel */
  int64_t staging_bytes, scratch_bytes;
  int64_t flag_bytes;         /* transfer and completion flags, one 128-byte line each */
  int64_t table_bytes;
  double compile_ms[6];       /* verify, DAG, fusion, schedule, workgroup allocation, lowering */
  int32_t opcode_hist[16];    /* lowered instructions by opcode bits (see ccl_instr_info.opcode) */
  int32_t specialized_instructions; /* generated kernel: instructions over its distinct sequences */
  int32_t specialized_waves_per_simd; /* generated kernel: minimum waves per SIMD it was compiled for
                                         (what its grid needs to be co-resident; 1 = no request) */
  int64_t specialized_code_bytes;   /* generated kernel: size of its code object */
  /* Parallelism of the fused instruction DAG of the base program (instance 0, all ranks;
     MSCCLang report, section 3.3: the analysis reports the instruction DAG's parallelism):
     dag_width = the most instructions no two of which are ordered by a dependency (a
     maximum antichain; -1 if the DAG is too large to compute it), dag_depth = the
     instructions on its longest dependency chain. */
  int32_t dag_width;
  int32_t dag_depth;
  /* generated kernel: 1 if every step reads its instruction record through the scalar
     cache (straight-line code whose pieces are all at most 8 KiB, 3 KiB under the LL
     protocol), 0 if each workgroup first copies its records into LDS */
  int32_t specialized_scalar_records;
} ccl_plan_info_t;

int ccl_plan_info(const ccl_plan* plan, ccl_plan_info_t* info);

/*
 * Algorithmic HBM bytes one ccl_execute moves for `count`: for every instruction,
 * (operands read + destinations written) x elements x element size, summed over
 * all instances and ranks. Returns a negative status on error.
 */
int64_t ccl_plan_bytes(const ccl_plan* plan, int64_t count);

/* One lowered instruction, for inspection and tests. opcode bits: */
#define CCL_I_RECV 0x1 /* first operand is the incoming transfer's staging slot */
#define CCL_I_SRCB 0x2 /* a second, local operand is added (reduce) */
#define CCL_I_DSTA 0x4 /* the result is stored to a local buffer */
#define CCL_I_SEND 0x8 /* the result is stored to the outgoing transfer's staging slot (or, direct
                          transport, straight into the receiver's buffer) */
#define CCL_I_LOCAL_IN 0x10 /* with CCL_I_RECV: the data was written into the local first operand by the
                               sender (direct transport); the receive waits for the flag, then reads it */
#define CCL_I_SKIP 0x20     /* a CCL_I_LOCAL_IN receive that stores nothing, sets no completion flag and
                               precedes nothing in the dependency graph: not executed (the end of the
                               launch makes its sender's stores visible) */
#define CCL_I_NOFLAG 0x40   /* a send whose receive is CCL_I_SKIP: no flag, no wait for its stores */

typedef struct {
  int32_t rank, wg, subpipe, channel, instance;
  int32_t opcode;
  int32_t a_buf, a_idx; /* local first operand (when not CCL_I_RECV) */
  int32_t b_buf, b_idx;
  int32_t d_buf, d_idx;
  int32_t count;        /* chunks */
  int32_t recv_peer, send_peer; /* -1 if none */
  int32_t xin, xout;    /* transfer ids, -1 if none */
  int32_t nwaits;       /* completion waits on other workgroups before the first slice */
  int32_t chunk_id;     /* chunk the scheduler attributes the task to */
  int32_t done_flag;    /* >= 0 if other workgroups wait for this instruction */
} ccl_instr_info;

/* Copy up to `cap` lowered instructions (ordered by workgroup, then execution
 * order) into `out`; *n receives the total number. */
int ccl_plan_export(const ccl_plan* plan, ccl_instr_info* out, size_t cap, size_t* n);

/*
 * Host-side check of the lowered plan: run every workgroup's instruction list
 * on symbolic values (multisets of contributing input elements) under the flag
 * protocol, in `nsims` seeded random interleavings at slice granularity, with
 * a small element count. Reports INVALID_PROGRAM if some interleaving deadlocks
 * or ends with an output that violates the collective's postcondition.
 */
int ccl_plan_check(const ccl_plan* plan, uint64_t seed, int nsims);

/* After the plan's last launch: CCL_OK, or CCL_ERR_TIMEOUT if a watchdog fired (the
 * error is then cleared; that launch's outputs are invalid). Synchronizes with the
 * plan's last launch. */
int ccl_plan_status(ccl_plan* plan);

/* Per-workgroup trace of the last launch of a CCL_FLAG_TRACE plan: for each
 * workgroup four uint64 values {first instruction start, last instruction end,
 * ticks spent waiting on flags, instructions run}, ticks of the 100 MHz device
 * wall clock. `bytes` must hold num_workgroups * 32; if it holds
 * (num_workgroups + num_instructions) * 32, four more values follow for every
 * lowered instruction in ccl_plan_export order {start, first slice's data ready,
 * end, 0}. */
int ccl_plan_read_trace(ccl_plan* plan, void* host, size_t bytes);

/*
 * Communication-link utilisation of the last launch of a CCL_FLAG_TRACE plan (MSCCLang
 * report, section 3.3: the analysis reports how busy the communication links are). A
 * connection is one (sending rank, receiving rank, channel, instance); it is busy while
 * an instruction that sends on it runs (from its start to its end in the device trace).
 * busy_fraction = length of the union of those intervals / the launch's span (first
 * workgroup start to last workgroup end). Fills up to `cap` records, ordered by
 * (src_rank, dst_rank, channel, instance); *n receives the number of connections.
 * Synchronizes with the plan's last launch. Errors: INVALID_ARGUMENT (no trace, null
 * pointers, no launch yet), HIP.
 */
typedef struct {
  int32_t src_rank, dst_rank, channel, instance;
  double busy_fraction;
} ccl_link_busy;

int ccl_plan_link_busy(ccl_plan* plan, ccl_link_busy* out, size_t cap, size_t* n);

/* ---- tuner (AutoCCL report, "Methods" 1-2: resource parameters tuned by
 * coordinate descent inside each implementation subspace) ----------------
 *
 * Two entry points instead of one: ccl_tune_coordinate_descent is the search alone
 * over any objective (pure host logic, testable without a GPU), ccl_tune plugs in the
 * device objective. ccl_tune takes a list of programs, one per algorithm subspace (the
 * pages' implementation dimension: e.g. ring and tree AllReduce), instead of one
 * program, so the parallel factor is a coordinate of the returned point rather than a
 * separate output, and it takes a base configuration whose dtype, max_count, scheduler,
 * allocation and kernel flags every candidate plan inherits. */
typedef struct {
  int32_t variant;         /* algorithm subspace (index into the program list) */
  int32_t parallel_factor; /* channels / instances (nc) */
  int32_t nthreads;        /* threads per workgroup (nt) */
  int32_t slice_bytes;     /* chunk size of one pipelined step (c) */
  int32_t protocol;        /* 0 = slice flags, 1 = low-latency units (CCL_FLAG_LL), 2 = slice flags with
                              direct transport (CCL_FLAG_DIRECT), 3 = 2 with non-temporal local traffic
                              (CCL_FLAG_DIRECT | CCL_FLAG_STREAMING) */
  int32_t reserved;
} ccl_tune_point;

typedef struct {
  const int32_t* factors;  int32_t nfactors;  /* ascending candidate values */
  const int32_t* nthreads; int32_t nnthreads;
  const int32_t* slices;   int32_t nslices;
  int32_t nvariants;       /* algorithm subspaces 0..nvariants-1 */
  int32_t warmup, iters;   /* per device evaluation */
  int32_t protocols;       /* protocol subspaces to search, bit p = protocol p of ccl_tune_point (0 = bit 0) */
} ccl_tune_space;

typedef struct {
  int32_t evaluations;     /* objective evaluations made */
  int32_t reserved;
  double best_score;       /* objective at the returned point (higher is better) */
  double start_score;      /* objective at the starting point */
} ccl_tune_report;

/* Objective: higher is better; a negative value marks an infeasible point. */
typedef double (*ccl_tune_objective)(const ccl_tune_point* point, void* user);

/*
 * Subspace coordinate descent (AutoCCL report, methods 1-2): for every (variant,
 * protocol) subspace, starting from the smallest candidate of each coordinate (or
 * from `start` where it lies in the space), optimize parallel_factor, then
 * nthreads, then slice_bytes; each coordinate is stepped up through its ascending
 * candidates while the objective improves, looking one candidate past a step that
 * does not improve before stopping. Passes repeat (at most four per subspace) until
 * one moves no coordinate; after the first, a coordinate that cannot rise is
 * stepped down the same way. Each point is evaluated at most once per subspace.
 * The best point over all subspaces is returned. Pure host logic.
 */
int ccl_tune_coordinate_descent(const ccl_tune_space* space, const ccl_tune_point* start,
                                ccl_tune_objective objective, void* user, ccl_tune_point* best,
                                ccl_tune_report* report);

/*
 * Tune on the device: variants[v] is the program of subspace v (all with the same
 * collective and nranks). Each evaluation creates a plan from `base` with the
 * point's (k, nt, slice), runs space->warmup untimed and space->iters timed
 * executions on `stream` over buffers the tuner allocates itself, and scores
 * the algorithmic bus bandwidth. Returns the best point and its report.
 */
int ccl_tune(const ccl_program_desc* const* variants, int nvariants, int64_t count,
             const ccl_plan_config* base, const ccl_tune_space* space, void* stream,
             ccl_tune_point* best, ccl_tune_report* report);

/* ---- measurement helper -------------------------------------------------- */
/* Plain 16-byte-vector device copy of `bytes` (multiple of 16) from src to dst
 * with `nblocks` x `nthreads`: the practical HBM streaming ceiling beside the
 * nominal 8 TB/s, and the reference kernel for calibrating traffic counters. */
int ccl_copy_probe(void* dst, const void* src, size_t bytes, int nblocks, int nthreads, void* stream);

/*
 * Message-passing litmus test of the transfer-store policy across workgroups (a
 * diagnostic beside the executor, like the copy probe). Eight producer workgroups
 * (ids 0-7) each hand `rounds` rounds of `words` fresh 32-bit words (a multiple of 4,
 * at most 2^20) to a consumer workgroup: id p + 8 (ids congruent mod 8: the same XCD
 * under the round-robin dispatch) or, with cross_xcd, id 8 + (p + 1) mod 8 (another
 * XCD). Each round uses the executor's own operations: plain data stores, the flag set
 * with a plain store when the consumer published the producer's XCD and with an
 * agent-scope release otherwise, agent-scope flag polls and agent-coherent data loads;
 * the consumer checks every word and acknowledges the round. Every wait is bounded by
 * timeout_us; a mismatch or an expiry stops every pair. The call allocates its own
 * device buffers, runs on `stream` and synchronizes with it. results (host, 64 values)
 * holds per pair p at [8p ...]: producer XCD, consumer XCD, rounds the consumer
 * completed, mismatching words, first mismatching round (0: none), its first word
 * index, flags set with a plain store, waits that expired.
 */
int ccl_litmus_message_passing(int cross_xcd, int rounds, int words, int64_t timeout_us, int64_t* results,
                               void* stream);

/*
 * Hop-latency probe (a diagnostic beside the executor, like the copy probe): the cost
 * of one hand-off of the executor in isolation, the unit of a latency-bound chain such
 * as the ring AllReduce's 2(P-1) dependent steps (MSCCLang report, section 3.1: a
 * receive-reduce-send step waits for the previous rank's send). A chain of hops + 1
 * workgroups on one XCD (ids 0, 8, 16, ...; the grid's other workgroups exit at once)
 * passes `bytes` (a multiple of 16, at most 4 MiB) of fp32 data along: workgroup 0
 * copies a source region into the first hand-off region, and every later workgroup
 * runs the executor's own slice code on it (flag poll by one thread, agent-coherent
 * loads, an added second operand of zeros when two_operands is set, XCD-local plain
 * stores into the next region), waits for its stores and sets its flag as a send does.
 * hops: 1..31 (the chain fits one XCD's 32 compute units at any workgroup size);
 * nthreads: a multiple of 64 in 64..1024; launches: 1..1000, each with new data and a
 * new epoch; every wait is bounded by timeout_us. ll: the hand-offs use the low-latency
 * protocol instead (run_ll: workgroup 0 writes flagged 8-byte units, each later one polls
 * the units it consumes and writes units for the next, the last writes plain data; no
 * flag stores or acknowledgement waits; timing from workgroup 0's start, so the per-hop
 * figure includes that first send and the last plain store: difference two hop counts
 * for the hand-off alone). window_bytes 0: every launch reuses the same lines, which
 * stay in the L2 between launches; otherwise (from twice a hand-off region, i.e. twice
 * the payload, or four times under LL, up to 16 MiB) every region owns a window of that
 * size and each launch moves its region one region further through it, so a launch
 * finds lines that recent launches did not touch, as a collective over buffers larger
 * than the L2 does.
 * us_per_hop (host, `launches` values): per launch, the wall-clock time from workgroup
 * 0's flag store to the last workgroup's acknowledged stores, divided by hops.
 * info (host, 4 values): [0] chain workgroups that ran on another XCD than workgroup 0,
 * summed over launches; [1] launches in which a wait expired (the probe stops there);
 * [2] launches whose last region differs from their source; [3] launches completed.
 * The call allocates its own device buffers, runs on `stream` and synchronizes with it
 * after every launch.
 */
int ccl_hop_probe(int hops, int bytes, int two_operands, int ll, int nthreads, int launches, int64_t window_bytes,
                  int64_t timeout_us, double* us_per_hop, int64_t* info, void* stream);

/* ---- compute-unit reservation (AutoCCL report, method 3 and its interference
 * results: communication tuned while computation runs beside it; ReSCCL report,
 * section 1: thread blocks the collective takes from computation) -------------- */

/*
 * Create a stream whose kernels run only on the compute units enabled in `mask`
 * (nwords 32-bit words, bit i = compute unit i of the device's numbering, 1..64 words;
 * bits beyond the device's CU count are ignored). Default priority. A plan created with
 * num_cus = the number of enabled CUs is checked for co-residency against them, so its
 * launches on this stream never wait for workgroups that cannot be placed; work on a
 * stream with the complementary mask never takes those CUs. The caller destroys the
 * stream with ccl_stream_destroy. Errors: INVALID_ARGUMENT (null pointers, bad length,
 * a mask that enables none of the device's CUs), HIP.
 */
int ccl_stream_create_cu_masked(const uint32_t* mask, int nwords, void** stream);
int ccl_stream_destroy(void* stream);

/*
 * Placement probe: launches `nblocks` one-wave workgroups on `stream`, each recording the
 * XCD it ran on and its hardware id word (gfx9 HW_ID: CU id bits 11:8, shader array bit
 * 12, shader engine bits 15:13) and holding its compute unit for hold_us microseconds, so
 * the set of (XCD, engine, array, CU) seen covers the CUs the stream may use. out (host)
 * receives 2 * nblocks values {XCD, HW_ID} in block order. Synchronizes with `stream`.
 */
int ccl_cu_probe(void* stream, int nblocks, int hold_us, uint32_t* out);

/* ---- errors --------------------------------------------------------------- */
const char* ccl_error_string(int status);
const char* ccl_last_error_detail(void);
int ccl_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CCL_H */
