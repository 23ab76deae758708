/* tk.h -- C ABI of libtk: one persistent, grid-resident HIP kernel per
 * functional training step on MI355X (gfx950).
 *
 * The operations mirror the execution boundary of the trainkernel pages
 * (trainkernel runtime.py: `compile_program`, `CompiledProgram.allocate`,
 * `run_into`, `__call__`, `resource_usage`, `ExecutionBuffers`) and the
 * generator's statistics (codegen.py: `GeneratedKernel`).
 *
 * Conventions for every entry point:
 *   - Return a tk_status; on anything but TK_OK, tk_last_error() holds a
 *     message ("tk: ...") for the calling thread.  Nothing is launched and no
 *     caller memory is written when a check fails.
 *   - Tensors are caller-owned views (tk_tensor); libtk never frees them.
 *     Sizes and strides are in elements.  Device pointers must be memory of
 *     the program's device.
 *   - Programs are immutable after tk_compile and may be used from several
 *     threads and streams at once given distinct output and workspace
 *     buffers (trainkernel runtime.py, class `CompiledProgram`: each call
 *     gets buffers of its own, which is what makes concurrent streams safe).
 */
#ifndef TK_H
#define TK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TK_F32 = 0, TK_F16 = 1, TK_BF16 = 2, TK_I8 = 3 } tk_dtype;

typedef enum {
  TK_OK = 0,
  TK_E_ARG = 1,          /* null pointer, bad option value, malformed call */
  TK_E_PARSE = 2,        /* program text does not parse */
  TK_E_UNSUPPORTED = 3,  /* op, dtype, layout or size outside the supported subset */
  TK_E_SHAPE = 4,        /* shape mismatch (program or buffer) */
  TK_E_STRIDE = 5,       /* stride / contiguity mismatch */
  TK_E_DTYPE = 6,        /* dtype mismatch */
  TK_E_DEVICE = 7,       /* wrong device, not gfx950, or no device for a run */
  TK_E_ALIAS = 8,        /* buffers overlap where they must not */
  TK_E_WORKSPACE = 9,    /* workspace too small, misaligned, or on the wrong device */
  TK_E_COUNT = 10,       /* wrong number of inputs / outputs */
  TK_E_HIP = 11,         /* a HIP runtime call failed (message has the HIP error) */
  TK_E_ABORTED = 12      /* an earlier launch of this program stopped at a grid barrier
                            that timed out (see tk_run_into) */
} tk_status;

/* A caller-owned tensor view.  `storage_base`/`storage_bytes` give the whole
 * allocation the view lives in (used for the aliasing rules, like storage
 * identity in the pages' `run_into`); when storage_base is NULL the view's own
 * extent is used. */
typedef struct {
  void* data;
  int32_t dtype;          /* tk_dtype */
  int32_t ndim;           /* 0..8 */
  int64_t shape[8];
  int64_t strides[8];     /* elements */
  const void* storage_base;
  uint64_t storage_bytes;
  int32_t device;
  int32_t requires_grad;  /* nonzero: rejected as an in-place target */
} tk_tensor;

/* Compile options (the pages' `generate` keywords, codegen.py).  Zero-filled
 * means defaults; tk_default_options fills the documented defaults. */
typedef struct {
  int32_t blocks_per_cu;       /* 1..8, default 1 (pages: blocks_per_sm) */
  int32_t max_blocks;          /* 0 = no cap */
  int32_t fuse_pointwise;      /* default 1: inline single-use pointwise values */
  int32_t fuse_epilogues;      /* default 1: fuse pointwise chains into GEMM tiles */
  int32_t inline_input_casts;  /* default 1 */
  int32_t split_k_gemv;        /* default 1: one-row products use the split-K GEMV */
  int32_t threads_per_block;   /* must be 256 (4 wave64) or 0 */
  int32_t fuse_updates;        /* default 1: fold an in-place SGD update into its
                                  weight-gradient GEMM tile when proven safe */
  int32_t barrier_every_op;    /* debug: one op per stage */
  int32_t num_cus;             /* plan-only compiles: CU count to plan for (0: 256) */
  int32_t gemm_split_k;        /* 0: automatic; else force split-K parts for MFMA GEMMs */
  int32_t force_grid;          /* 0: automatic; else launch exactly this many workgroups
                                  (clamped to the co-resident capacity) */
  int32_t launch_mode;         /* 0 (default): cooperative launch (co-residency guaranteed by
                                  the runtime, or the launch fails).  1: ordinary launch of a
                                  grid the compiler sized to be co-resident on an idle device
                                  (occupancy x CUs); avoids the runtime's serialization of
                                  cooperative launches.  If other work keeps a CU busy, the
                                  grid barrier's bounded wait turns a stall into an abort
                                  (tk_workspace_status), never a hang. */
  int32_t gemm_tile;           /* 0: automatic; 1: force 128x128 MFMA tiles; 2: force 64x64 */
  int32_t batch_epilogues;     /* 0 (default): a contraction tile whose epilogue program is short
                                  and simple runs it from registers, and a column sum whose source
                                  is one load reads its rows straight into registers; 1: every
                                  epilogue and reduction source runs on the expression machine's
                                  batches (same partitions, same results, bit for bit) */
  int32_t colsum_fusion;       /* column sums of a contraction's B operand (a bias gradient
                                  summed from the gradient its weight-gradient product reads)
                                  computed by that product's first tile row: 0 (default) where
                                  the reduction's own items would add a round of items to its
                                  stage (and K <= 512 unless K is a multiple of 64); 1 wherever
                                  legal; -1 never */
} tk_options;

/* Plan and kernel statistics (pages: `GeneratedKernel` and `resource_usage`). */
typedef struct {
  uint64_t workspace_bytes;      /* bytes the workspace must hold (header + arena) */
  int32_t n_stages;
  int32_t grid_barriers;         /* n_stages - 1 */
  int32_t materialized_ops;
  int32_t inlined_ops;
  int32_t fused_epilogues;       /* GEMM/GEMV tiles carrying a pointwise chain */
  int32_t side_epilogues;
  int32_t fused_updates;
  int32_t matrix_core_ops;       /* contractions on MFMA */
  int32_t direct_outputs;        /* values written straight into caller outputs */
  int32_t direct_state_commits;  /* in-place outputs written straight into inputs */
  int32_t staged_commits;
  int32_t grid_size;             /* workgroups per launch */
  int32_t max_work_items;
  int32_t num_cus;
  int32_t blocks_per_cu;         /* resident workgroups per CU used */
  int32_t occupancy;             /* max resident workgroups per CU (0 in plan-only mode) */
  int32_t vgprs, sgprs, lds_bytes, scratch_bytes;
  int32_t n_tasks;
  int32_t reserved[5];
} tk_stats;

typedef struct tk_program tk_program;

/* Allocator callback for tk_allocate: returns `bytes` of device memory on
 * `device` owned by the caller (NULL on failure).  `bytes` may be 0. */
typedef void* (*tk_alloc_fn)(void* ctx, uint64_t bytes, int32_t device);

void tk_default_options(tk_options* opts);

/* Parse and validate a `tkir 1` program, schedule it and upload its plan.
 * device >= 0: that device must be gfx950; its CU count and the kernel's
 * occupancy size the grid.  device == -1: plan only (no HIP calls at all); the
 * program can be queried, dumped and validated against, but not run.
 * Rejections follow the pages' generator and compile_program: non-finite
 * scalars, unsupported ops/dtypes, bad shapes/strides/broadcasts, invalid
 * in-place maps, option ranges. */
tk_status tk_compile(const char* ir, size_t ir_len, const tk_options* opts, int32_t device, tk_program** out);

tk_status tk_query(const tk_program* prog, tk_stats* out);

/* Write a human-readable schedule (stages, tasks, arena) into buf (always
 * NUL-terminated when len > 0).  *needed receives the full length + 1. */
tk_status tk_dump_plan(const tk_program* prog, char* buf, size_t len, size_t* needed);

/* Copy the device plan (the bytes tk_compile uploads: a DHeader, the DStage
 * table and one descriptor blob per stage, laid out as in csrc/plan.h) into
 * buf, at most len bytes.  *needed receives the plan's size.  For tools that
 * check a schedule on the host (the schedule race checker). */
tk_status tk_plan_bytes(const tk_program* prog, void* buf, size_t len, size_t* needed);

/* Fill `outputs` (n_out descriptors) and `workspace` for a run on `inputs`
 * (pages: `allocate`).  In-place output slots receive their input's own
 * descriptor; other outputs and the workspace come from `alloc` (contiguous,
 * the program's output dtype/shape).  The workspace header is initialised on
 * `stream` (synchronously before return). */
tk_status tk_allocate(const tk_program* prog, const tk_tensor* inputs, size_t n_in, tk_alloc_fn alloc, void* ctx,
                      tk_tensor* outputs, size_t n_out, tk_tensor* workspace, void* stream);

/* Run every check of tk_run_into without touching the GPU (pages:
 * `_validate_inputs` and the buffer checks of `run_into`): counts; each input's
 * device, dtype, shape and exact strides; each output's device, dtype, shape
 * and contiguity; workspace device, size (>= workspace_bytes), 256-byte
 * alignment; in-place slots bound to their declared input with identical
 * strides; in-place targets not aliased by another input and not
 * requires_grad; outputs and workspace pairwise disjoint and disjoint from all
 * inputs except declared in-place targets. */
tk_status tk_validate_into(const tk_program* prog, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                           size_t n_out, const tk_tensor* workspace);

/* Validate, then launch the step on `stream` (a hipStream_t, NULL = default
 * stream) and return without waiting (pages: `run_into`).  One cooperative
 * launch; every stage ends in a global-memory grid barrier.  The workspace
 * header must have been initialised once (tk_allocate or tk_workspace_init);
 * it stays valid across launches.  Reuse of outputs/workspace must be ordered
 * by the caller; calls overlapping on one workspace race.
 * Every wait at a grid barrier is bounded.  A launch whose barrier times out
 * stops (its outputs and in-place targets are then partly written), marks its
 * workspace aborted and records that in host memory the program owns; from
 * then on tk_run_into returns TK_E_ABORTED before any check or launch, and a
 * launch on the aborted workspace runs nothing, until tk_workspace_init
 * re-initialises the workspace.  The launch that timed out itself returned
 * TK_OK (the error is detected asynchronously): tk_workspace_status reports
 * it after synchronising the stream. */
tk_status tk_run_into(const tk_program* prog, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                      size_t n_out, const tk_tensor* workspace, void* stream);

/* tk_run_into without a workspace argument and without allocating anything:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * step runs in the library's own workspace, a static device array of
 * TK_STATIC_WORKSPACE_BYTES (128 MiB) per device, held from the first call
 * on a device until the process ends; programs whose workspace_bytes
 * exceed it are rejected with TK_E_WORKSPACE before anything else is
 * checked (use tk_run_into).  Every call first clears the workspace header
 * (barrier flags, epochs, abort word) with a small fill kernel on `stream`,
 * then launches; the arena keeps whatever the last call left.  All calls on
 * one device share that one workspace: calls that overlap on a device (on
 * different streams, or from different threads without ordering) race.
 * Inputs and outputs are checked as in tk_run_into.  When an earlier launch
 * of the program stopped at a timed-out barrier, the call returns
 * TK_E_ABORTED once (nothing launched) and clears that record. */
#define TK_STATIC_WORKSPACE_BYTES (128ull << 20)
tk_status tk_run_into_noalloc(const tk_program* prog, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                              size_t n_out, void* stream);

/* Zero the workspace header (barrier state, abort flag) on `stream` with a
 * small kernel (safe under graph capture), and clear the program's record of
 * an aborted launch (TK_E_ABORTED). */
tk_status tk_workspace_init(const tk_program* prog, const tk_tensor* workspace, void* stream);

/* Synchronise `stream` and read the workspace header: *aborted = 1 when a
 * launch stopped at a timed-out barrier (*stage = the stage it stopped in). */
tk_status tk_workspace_status(const tk_tensor* workspace, void* stream, int32_t* aborted, int32_t* stage);

/* Debug/measurement switches for subsequent launches of this program:
 * timestamps (workgroup 0 records arrival/departure ticks of every barrier in
 * the workspace header), stagger_seed (nonzero: every workgroup sleeps a seeded
 * pseudo-random time before each work item), deadline_ticks (barrier wait
 * limit in 100 MHz ticks; 0 restores the default of 4 s). */
tk_status tk_set_debug(tk_program* prog, int32_t timestamps, uint32_t stagger_seed, uint64_t deadline_ticks);

/* Copy the per-stage barrier timestamps (2 * n_stages u64, arrival and
 * departure of workgroup 0, 100 MHz ticks) out of a workspace (synchronises
 * `stream`). */
tk_status tk_read_timestamps(const tk_program* prog, const tk_tensor* workspace, void* stream, uint64_t* out,
                             size_t n);

/* Free the program's device plan and host memory (the counterpart of
 * tk_compile; trainkernel runtime.py holds a compiled program as an object
 * that owns its loaded kernel).  NULL is ignored.  No launch of the program
 * may still be running; caller tensors are never touched. */
void tk_destroy(tk_program* prog);

/* Thread-local message ("tk: ...") of the last failed call on this thread.
 * The messages name the failed check the way trainkernel runtime.py's
 * `run_into` and `_validate_inputs` do (e.g. "incorrect output buffer
 * count", "inplace target must not alias another input"). */
const char* tk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TK_H */
