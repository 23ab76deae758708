// Device-resident plan of one compiled whole-step program.
//
// The host scheduler (tk_sched.cpp) turns a program into a list of stages;
// the persistent kernel (tk_device.hip) walks the stages, runs every work item
// of a stage, and separates consecutive stages with one grid barrier.  This
// header is the contract between the two: plain structs, no pointers (bases are
// slots filled per launch), identical layout on host and device.
//
// The pages' generator (trainkernel codegen.py, `_Generator.generate`) emits one
// straight-line kernel per program with a grid sync between dependent
// operators; here the same schedule is data, interpreted by one AOT-compiled
// kernel, so nothing is compiled at run time.
#pragma once
#include <stdint.h>

namespace tkplan {

enum DType : uint8_t { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 };

constexpr int kBlock = 256;         // threads per workgroup (4 wave64)
constexpr int kMaxBases = 240;      // pointer slots per launch (inputs, outputs, workspace)
constexpr int kMaxDims = 4;         // iteration dims after collapsing
constexpr int kMaxSlots = 3;        // saved values in the expression machine (LDS-resident)
constexpr uint32_t kPlanLds = 16384;       // LDS bytes for the current stage's descriptors (every stage blob fits)
constexpr uint32_t kMaxGrid = 1024;        // workgroups per launch (barrier flag slots)
constexpr uint32_t kHdrArrive = 16384;     // u32 [kMaxGrid] arrival epochs, one per workgroup
constexpr uint32_t kHeaderBytes = kHdrArrive + kMaxGrid * 4;  // 20480: header size
constexpr uint32_t kMaxTimedStages = 400;
// The library's own per-device workspace for callers that cannot allocate
// (tk_run_into_noalloc): header plus arena of at most this many bytes.
constexpr uint64_t kStaticWorkspaceBytes = 128ull << 20;

// Workspace header layout (bytes).  Each word sits on its own 64-byte line.
constexpr uint32_t kHdrEpoch = 0;      // last barrier epoch of the previous launch on this workspace
constexpr uint32_t kHdrGen = 64;       // (unused)
constexpr uint32_t kHdrAbort = 128;    // nonzero: a barrier timed out; the launch stopped
constexpr uint32_t kHdrAbortStage = 192;
constexpr uint32_t kHdrStamps = 1024;  // optional: u64 [stage][4] of workgroup 0: stage start, items done,
                                       // barrier entry, barrier exit (100 MHz ticks)

// Addressing of one operand over a task's iteration space: element
// (c0..c3) lives at bases[base] + (offset + sum c_i * stride[i]) * size(dtype).
struct DView {
  int64_t offset;
  int64_t stride[kMaxDims];
  uint16_t base;
  uint8_t dtype;
  uint8_t pad[5];
};
static_assert(sizeof(DView) == 48, "DView layout");

// Expression machine.  One accumulator vector (W elements per thread), a few
// saved slots; each instruction reads the accumulator and at most one other
// operand (a view load, a scalar, or a slot) and optionally rounds its result
// to a storage dtype (round-to-nearest-even), as every pointwise op of the
// pages rounds to its output dtype.
enum VmOp : uint8_t {
  VM_LOAD = 1,   // acc = operand
  VM_ADD,        // acc = acc + a*x        (rev: x + a*acc)
  VM_SUB,        // acc = acc - a*x        (rev: x - a*acc)
  VM_MUL,        // acc = acc * x
  VM_DIV,        // acc = acc / x          (rev: x / acc)
  VM_NEG,        // acc = -acc
  VM_RELU,       // acc = acc < 0 ? 0 : acc
  VM_SQUARE,     // acc = acc * acc
  VM_POW,        // acc = powf(acc, a)
  VM_TB,         // threshold_backward: rev=0: (x <= a) ? 0 : acc ; rev=1: (acc <= a) ? 0 : x
  VM_SAVE,       // slot[arg] = acc
  VM_STORE,      // view[arg] = acc (converted to the view's dtype)
  VM_SCALE,      // acc = a * acc (addmm alpha)
  VM_ZERO,       // acc = 0
  VM_SQRT,       // acc = sqrt(acc), correctly rounded
};
enum VmSrc : uint8_t { SRC_NONE = 0, SRC_VIEW = 1, SRC_SCALAR = 2, SRC_SLOT = 3 };
constexpr uint8_t RND_NONE = 0xff;

struct DIns {
  uint8_t op;
  uint8_t src;
  uint8_t rnd;   // dtype to round the result to, or RND_NONE
  uint8_t rev;
  uint16_t arg;  // view index (SRC_VIEW / VM_STORE) or slot index
  uint16_t pad;
  float a;       // alpha, threshold or exponent
  float s;       // scalar operand (SRC_SCALAR)
};
static_assert(sizeof(DIns) == 16, "DIns layout");

enum TaskKind : uint8_t {
  T_EW = 1,        // elementwise expression over an iteration space
  T_GEMM_MFMA,     // tiled contraction on matrix cores (bf16/f16 operands)
  T_GEMM_SIMT,     // tiled contraction with fp32 FMA (any dtypes)
  T_GEMM_REDUCE,   // split-K: sum partial tiles in fixed order, then epilogue
  T_GEMV_Q8,       // one-row product with an int8 blockwise-scaled weight
  T_GEMV,          // one-row product with a float weight
  T_RED_ROWS,      // reduce trailing iteration dims (rows x R)
  T_RED_COLS,      // reduce leading iteration dims (R x cols)
  T_RED_FINAL,     // combine per-part partials in fixed order, then epilogue
};

// Flags
constexpr uint32_t F_MEAN = 1u;        // divide the sum by `count`
constexpr uint32_t F_PARTIAL = 2u;     // write fp32 partials to scratch instead of finishing
constexpr uint32_t kGemvRows = 4;      // int8-weight products: activation rows per work item (a slab)
constexpr uint32_t F_ROWWG = 4u;       // combine: one workgroup per output, parts summed across its threads
constexpr uint32_t F_XQ = 32u;         // int8 GEMV: quantise the activation rows to Q8_0 (blocks of 32,
                                       //   d = amax/127, codes round(x/d)) and multiply codes by codes
constexpr uint32_t F_FASTEPI = 64u;    // contraction tile: the epilogue runs as a register program (at most
                                       //   kFastIns instructions, no slots, 2-D views with column stride 1
                                       //   or 0 and 8-element chunk alignment, at most kFastLoads loaded
                                       //   views, no load after a store that may overlap it)
constexpr uint32_t F_COLDIRECT = 128u;  // column reduction whose source program is one load of a 2-D view with
                                       //   column stride 1: rows are summed straight from memory, not in batches
constexpr uint32_t F_BSUM = 512u;       // contraction whose first tile row also sums its B operand over K per
                                       //   column and runs a fused column reduction's finishing program
constexpr uint32_t F_COLLANES32 = 256u;  // direct column reduction in one part: an item is 8 column chunks (64
                                        //   columns) x 32 row lanes instead of 32 chunks x 8 row lanes
constexpr int kFastIns = 8;
constexpr int kFastLoads = 3;
// Register epilogues: the unit-stride loaded views of a tile are copied into
// the top of the workgroup's LDS arena before the main loop starts, above the
// operand ring (16 bytes per 8-element chunk and plane; an fp32 view takes
// two planes).  Byte offsets within the arena:
constexpr uint32_t kArenaBytes = 131072;     // the workgroup's LDS arena
constexpr uint32_t kFastStage64 = 81920;     // 64x64 tiles (their operand ring ends at 64 KB)
constexpr uint32_t kFastStage128 = 98304;    // 128x128 tiles (their operand ring ends at 96 KB)
// A register epilogue's program is also encoded as one record per
// instruction, two DIns slots each, at fin_first (fin_len = 2 * instructions):
//   slot 0: the instruction itself; its pad field holds the byte offset / 16
//           of the view's staged chunks in the arena (0xffff: not staged);
//   slot 1: the instruction's view, resolved: op = src = 0, rnd = dtype,
//           rev = column stride (0 or 1), arg = base slot, a = offset bits,
//           s = row stride bits (32-bit element indices).
constexpr uint16_t kFastNotStaged = 0xffff;

struct DTask {
  uint8_t kind;
  uint8_t width;       // elements per thread chunk (8 or 1)
  uint8_t ndim;        // iteration dims
  uint8_t tile;        // GEMM tile code
  uint32_t flags;
  uint32_t n_items;    // work items of this task in its stage
  uint32_t item_begin; // first item index within the stage
  uint32_t expr_first; // expression program (instructions): element source,
  uint32_t expr_len;   //   or the epilogue of a contraction
  uint32_t fin_first;  // reductions: the finishing program (mean, rounding, store)
  uint32_t fin_len;
  uint32_t dims[kMaxDims];  // iteration shape (elementwise / reduction source / GEMM output [m, n])
  uint32_t dmul[kMaxDims];  // division by dims[d] (d >= 1): q = (t + ((e - t) >> min(l,1))) >> max(l-1,0),
  uint8_t dsh[kMaxDims];    //   t = mulhi(dmul[d], e), l = dsh[d] = ceil(log2 dims[d])  (Granlund-Montgomery)
  uint32_t m, n, k;         // contraction sizes; reductions: rows/cols and reduced size
  uint32_t split;           // split-K parts / reduction parts
  uint32_t kchunk;          // K elements per split part / rows per reduction part
  uint32_t tiles_m, tiles_n;
  uint16_t va, vb, vs, vx;  // operand views (A, B, scale, extra)
  uint64_t scratch;         // byte offset of fp32 partials in the workspace
  float count;              // mean divisor
  uint32_t group_m;         // contractions: tile rows per group of the tile order (see the kernel)
  uint32_t bs_first;        // F_BSUM: finishing program of the column sums of B (one element per column)
  uint32_t bs_len;
};
static_assert(sizeof(DTask) % 8 == 0, "DTask layout");

// A stage's descriptors form one contiguous blob in the plan:
// [DTask x n_tasks][DView x n_views][DIns x n_ins], indices local to the blob,
// so a workgroup can stage the whole blob in LDS before the stage starts.
struct DStage {
  uint32_t blob_off;    // bytes from the plan start (16-byte aligned)
  uint32_t blob_bytes;  // multiple of 16
  uint32_t n_tasks;
  uint32_t n_items;
  uint32_t off_views;   // bytes from the blob start
  uint32_t off_ins;
  uint32_t n_views;
  uint32_t n_ins;
};

struct DHeader {
  uint32_t magic;
  uint32_t n_stages;
  uint32_t off_stages;  // bytes from the plan start
  uint32_t bytes;
  uint32_t max_blob;    // largest stage blob
  uint32_t pad[3];
};
constexpr uint32_t kPlanMagic = 0x31706b74u;  // "tkp1"

// Kernel launch arguments (passed by value as the kernel argument block).
struct KArgs {
  const uint8_t* plan;
  uint8_t* ws;                 // workspace: header then arena
  uint64_t deadline_ticks;     // barrier wait limit (100 MHz ticks); 0 = default
  uint32_t flags;              // K_* debug switches
  uint32_t stagger_seed;
  uint32_t n_bases;
  uint32_t pad;
  uint32_t* host_abort;        // pinned host words [aborted, stage] of the program, or null
  void* bases[kMaxBases];
};
constexpr uint32_t K_TIMESTAMPS = 1u;
constexpr uint32_t K_STAGGER = 2u;

}  // namespace tkplan
