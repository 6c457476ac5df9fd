// Records the host compiler lowers a plan into and the executor kernel reads.
// Layout: a rank x workgroup x pipeline-order table (ReSCCL report, section 2.2,
// "lightweight kernel generation": rank, thread-block and pipeline dimensions),
// kept as data that one generic kernel interprets.
#pragma once
#include <stdint.h>

namespace ccl {

constexpr int kMaxRanks = 64;
constexpr int kNumBufs = 3;  // input, output, scratch

// Opcode bits of a lowered instruction (same values as CCL_I_* in ccl.h). With
// OPB_LOCAL_IN a receive's data is already in the local first operand, written there
// by the sender (direct transport); the receive only waits for the transfer's flag
// before reading it.
// OPB_SKIP marks such a receive that nothing depends on (it is not executed) and
// OPB_NOFLAG a send whose receiver is skipped (no flag, no wait for its stores).
// OPB_NOSYNC (LL plans) no later instruction of the workgroup touches a local chunk range
// this one writes or writes one it reads, and it sets no completion flag: its waves go
// on to the next instruction without a workgroup barrier.
enum : uint32_t {
  OPB_RECV = 1u, OPB_SRCB = 2u, OPB_DSTA = 4u, OPB_SEND = 8u, OPB_LOCAL_IN = 16u, OPB_SKIP = 32u, OPB_NOFLAG = 64u,
  OPB_NOSYNC = 128u
};
constexpr uint32_t kStagingBuf = 15u;  // DevExec::op target-buffer field: the staging pool

struct DevWG {  // one workgroup of the launch
  int32_t rank;
  int32_t first;  // first instruction in DevInstr[]
  int32_t n;      // number of instructions, run in order
  int32_t trace_slot;
};

struct DevInstr {  // host-side lowered instruction
  uint32_t op;     // OPB_* bits
  int32_t cnt;     // chunks covered
  int32_t a_buf, a_idx;  // local first operand (unless OPB_RECV)
  int32_t b_buf, b_idx;  // local second operand (OPB_SRCB)
  int32_t d_buf, d_idx;  // local destination (OPB_DSTA)
  int32_t xin, xout;     // transfer ids (OPB_RECV / OPB_SEND)
  int32_t wait_begin, nwaits;  // completion flags to await, in DevExec::waits
  int32_t done_flag;           // completion flag to set (-1 = none)
  int32_t instance;            // instance sub-chunk index (0..k-1)
  int32_t pad0;                // chunk index that fixes the instruction's element range
  int32_t peer_wg;             // OPB_SEND: launch-grid workgroup that receives (-1 = none)
  int32_t t_buf, t_rank, t_idx;  // direct OPB_SEND: receiver's buffer, rank and chunk (t_buf -1: staging slot)
  int32_t done_peer;             // done_flag >= 0: the one workgroup that waits for it (-1: several)
};

struct DevXfer {  // 32 bytes: one send -> recv transfer
  uint64_t slot_off;  // byte offset of its staging slot in the staging pool (256-aligned)
  int32_t phase_idx;  // chunk whose range start fixes the data's offset inside the slot (-1: none)
  int32_t instance;
  int32_t cnt;
  int32_t direct;     // 1: written straight into the receiver's buffer, no slot
  int32_t pad1, pad2;
};

// What the kernel reads for one lowered instruction at one element count: the
// opcode, buffers, transfer and completion-flag ids, and the byte offsets of every
// operand (inside the rank's buffer, or inside the staging pool for slots, in-slot
// phase included), its length and slice count. Built on the host from DevInstr and
// the count when a count is first used, cached on the device, and copied into LDS by
// each workgroup at launch.
struct DevExec {  // 80 bytes
  // OPB_* bits | a_buf << 8 | b_buf << 12 | d_buf << 16 | t_buf << 20 | t_rank << 24, where
  // t_buf / t_rank name the receiver's buffer of a direct send (t_buf kStagingBuf: a slot)
  uint32_t op;
  int32_t xin, xout, done_flag;
  int32_t wait_begin, nwaits;
  int32_t nsl;     // slices (simple protocol)
  int32_t peer_wg; // OPB_SEND: launch-grid workgroup of the receiver (-1 = none)
  int64_t len;     // elements
  int64_t a_off, b_off, d_off, t_off;
  // done_flag >= 0: launch-grid workgroup of the only waiter (-1: several); a waiter on
  // the producer's XCD (its tag says so) lets an XCD-local layout skip the L2 writeback
  int32_t done_peer;
  int32_t pad1;
};
static_assert(sizeof(DevExec) == 80, "DevExec layout");

// Transfer and completion flags each own a 128-byte cache line (this many 8-byte
// words apart): flags packed into shared lines put every writer and poller of a line
// in one queue of one L2 channel.
constexpr int kFlagStride = 16;

// Kernel arguments, passed by value.
struct ExecArgs {
  const DevWG* wgs;
  const DevExec* recs;
  const int32_t* waits;
  unsigned long long* xflags;  // per transfer (kFlagStride apart): epoch << 24 | slices completed
  unsigned long long* dflags;  // per completion flag (kFlagStride apart): epoch when done
  unsigned char* staging;
  unsigned int* err;           // [code, wg, instr, epoch_lo]
  unsigned long long* abort_word;  // epoch of an aborted launch
  unsigned long long* trace;   // 4 words per workgroup, or null
  int64_t slice_elems;         // slice length in elements (multiple of 64)
  unsigned long long epoch;    // launch number, >= 1
  long long timeout_ticks;     // watchdog budget per wait, device wall-clock ticks
  int32_t ll;                  // low-latency protocol: slots hold {4 data bytes, 4-byte flag} units
  uint32_t ll_flag;            // flag value of this launch's units (never 0)
  // Per launch-grid workgroup: epoch << 8 | 0x10 | XCD id, published at the start of
  // each launch. A sender whose receiver's entry names the sender's own XCD for this
  // launch sets the transfer's flag with a plain store; otherwise (or when null) with a
  // full agent-scope release.
  unsigned long long* xcd_tags;
  unsigned char* base[kNumBufs][kMaxRanks];  // per-rank buffer base pointers
};

constexpr unsigned long long kEpochShift = 24;  // slices per transfer < 2^24

}  // namespace ccl
