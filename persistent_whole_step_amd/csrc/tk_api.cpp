// C ABI of libtk (include/tk.h): compile, query, allocate, validate, run.
//
// The checks mirror the pages' execution boundary (trainkernel runtime.py,
// `compile_program`, `_validate_inputs`, `allocate`, `run_into`) with storage
// identity replaced by byte-range overlap of caller-described allocations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "tk_internal.hpp"

using namespace tkplan;

hipError_t tk_device_launch(const KArgs& ka, int grid, hipStream_t stream);
hipError_t tk_device_launch_resident(const KArgs& ka, int grid, hipStream_t stream);
hipError_t tk_device_occupancy(int* blocks_per_cu);
hipError_t tk_device_attributes(hipFuncAttributes* attr);
hipError_t tk_device_zero_header(uint8_t* ws, hipStream_t stream);
hipError_t tk_device_static_workspace(int device, void** out);

struct tk_program {
  tk::Plan plan;
  tk::Options opts;
  int device = -1;
  void* d_plan = nullptr;
  int grid = 1;
  uint32_t dbg_flags = 0;
  uint32_t stagger = 0;
  uint64_t deadline = 0;
  // Pinned, device-visible host words [aborted, stage]: a launch that stops at
  // a timed-out grid barrier (or finds its workspace already aborted) sets
  // them, so later tk_run_into calls report TK_E_ABORTED without waiting on
  // the device.  tk_workspace_init clears them.
  volatile uint32_t* h_abort = nullptr;
  uint32_t* d_abort = nullptr;
};

namespace {

thread_local std::string g_err;

tk_status fail(tk_status c, const std::string& m) {
  g_err = "tk: " + m;
  return c;
}

#define TK_TRY(body)                          \
  try {                                       \
    body                                      \
  } catch (const tk::Error& e) {              \
    g_err = e.what();                         \
    return e.code;                            \
  } catch (const std::exception& e) {         \
    g_err = std::string("tk: ") + e.what();   \
    return TK_E_ARG;                          \
  }

tk_status hip_fail(hipError_t e, const char* what) {
  return fail(TK_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t numel_of(const tk_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}

// Byte range a tensor occupies for aliasing rules.
std::pair<uintptr_t, uintptr_t> extent(const tk_tensor& t) {
  if (t.storage_base) {
    uintptr_t b = (uintptr_t)t.storage_base;
    return {b, b + t.storage_bytes};
  }
  int64_t n = numel_of(t);
  if (n == 0) return {0, 0};
  int64_t hi = 0;
  for (int i = 0; i < t.ndim; ++i) hi += (t.shape[i] - 1) * t.strides[i];
  uintptr_t b = (uintptr_t)t.data;
  return {b, b + (uintptr_t)((hi + 1) * tk::dtype_size((uint8_t)t.dtype))};
}

bool overlap(const tk_tensor& a, const tk_tensor& b) {
  if (numel_of(a) == 0 || numel_of(b) == 0) return false;
  auto x = extent(a), y = extent(b);
  return x.first < y.second && y.first < x.second;
}

bool contiguous(const tk_tensor& t) {
  int64_t expect = 1;
  for (int i = t.ndim - 1; i >= 0; --i) {
    if (t.shape[i] != 1 && t.strides[i] != expect) return false;
    expect *= t.shape[i];
  }
  return true;
}

bool matches_shape(const tk_tensor& t, const tk::Spec& s) {
  if (t.ndim != (int)s.shape.size()) return false;
  for (int i = 0; i < t.ndim; ++i)
    if (t.shape[i] != s.shape[i]) return false;
  return true;
}

void check_inputs(const tk_program* p, const tk_tensor* inputs, size_t n_in, int device) {
  const auto& pl = p->plan;
  if (n_in != pl.inputs.size())
    tk::raise(TK_E_COUNT, "expected " + std::to_string(pl.inputs.size()) + " inputs, got " + std::to_string(n_in));
  if (n_in && !inputs) tk::raise(TK_E_ARG, "inputs is NULL");
  for (size_t i = 0; i < n_in; ++i) {
    const tk_tensor& t = inputs[i];
    const tk::Spec& s = pl.inputs[i];
    if (t.device != device) tk::raise(TK_E_DEVICE, "input " + std::to_string(i) + " is on another device");
    if (t.dtype != s.dtype) tk::raise(TK_E_DTYPE, "input " + std::to_string(i) + " does not match the compiled dtype");
    if (!matches_shape(t, s)) tk::raise(TK_E_SHAPE, "input " + std::to_string(i) + " does not match the compiled shape");
    // Exact strides, except where no element is addressed through them
    // (size-1 dims and empty tensors).
    const bool empty = numel_of(t) == 0;
    for (int d = 0; d < t.ndim; ++d)
      if (!empty && t.shape[d] > 1 && t.strides[d] != s.strides[d])
        tk::raise(TK_E_STRIDE, "input " + std::to_string(i) + " does not match the compiled strides");
    if (numel_of(t) && !t.data) tk::raise(TK_E_ARG, "input " + std::to_string(i) + " has no data");
  }
  for (auto& kv : pl.inplace)
    if (inputs[kv.second].requires_grad) tk::raise(TK_E_ARG, "inplace targets must be detached from autograd");
}

void check_buffers(const tk_program* p, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs, size_t n_out,
                   const tk_tensor* ws, int device) {
  const auto& pl = p->plan;
  check_inputs(p, inputs, n_in, device);
  if (n_out != pl.outputs.size()) tk::raise(TK_E_COUNT, "incorrect output buffer count");
  if (n_out && !outputs) tk::raise(TK_E_ARG, "outputs is NULL");
  if (!ws) tk::raise(TK_E_ARG, "workspace is NULL");
  if (ws->device != device) tk::raise(TK_E_WORKSPACE, "workspace is on another device");
  if (ws->ndim != 1 || (uint64_t)ws->shape[0] * tk::dtype_size((uint8_t)ws->dtype) < pl.workspace_bytes)
    tk::raise(TK_E_WORKSPACE, "workspace does not match compiled requirements (" + std::to_string(pl.workspace_bytes) + " bytes)");
  if (ws->strides[0] != 1) tk::raise(TK_E_WORKSPACE, "workspace must be contiguous");
  if (!ws->data || ((uintptr_t)ws->data & 255)) tk::raise(TK_E_WORKSPACE, "workspace must be 256-byte aligned");
  for (size_t s = 0; s < n_out; ++s) {
    const tk_tensor& t = outputs[s];
    const tk::Spec& sp = pl.outputs[s];
    if (t.device != device) tk::raise(TK_E_DEVICE, "output " + std::to_string(s) + " is on another device");
    if (t.dtype != sp.dtype) tk::raise(TK_E_DTYPE, "output buffer does not match compiled requirements (dtype)");
    if (!matches_shape(t, sp)) tk::raise(TK_E_SHAPE, "output buffer does not match compiled requirements (shape)");
    if (!contiguous(t)) tk::raise(TK_E_STRIDE, "output buffer does not match compiled requirements (contiguity)");
    if (numel_of(t) && !t.data) tk::raise(TK_E_ARG, "output " + std::to_string(s) + " has no data");
    auto it = pl.inplace.find((int)s);
    if (it != pl.inplace.end()) {
      const tk_tensor& tgt = inputs[it->second];
      bool same_strides = t.ndim == tgt.ndim;
      for (int d = 0; same_strides && d < t.ndim; ++d)
        same_strides = t.shape[d] <= 1 || t.strides[d] == tgt.strides[d];
      if (t.data != tgt.data || !same_strides) tk::raise(TK_E_ALIAS, "inplace output must bind its declared input");
      for (size_t i = 0; i < n_in; ++i)
        if ((int)i != it->second && overlap(inputs[i], tgt))
          tk::raise(TK_E_ALIAS, "inplace target must not alias another input");
    }
  }
  // outputs + workspace pairwise disjoint; disjoint from inputs except an
  // in-place slot with its own target
  for (size_t a = 0; a <= n_out; ++a) {
    const tk_tensor& x = a < n_out ? outputs[a] : *ws;
    for (size_t b = a + 1; b <= n_out; ++b) {
      const tk_tensor& y = b < n_out ? outputs[b] : *ws;
      if (overlap(x, y)) tk::raise(TK_E_ALIAS, "execution buffers must not alias inputs or each other");
    }
    for (size_t i = 0; i < n_in; ++i) {
      if (!overlap(x, inputs[i])) continue;
      auto it = a < n_out ? pl.inplace.find((int)a) : pl.inplace.end();
      if (it != pl.inplace.end() && it->second == (int)i) continue;
      tk::raise(TK_E_ALIAS, "execution buffers must not alias inputs or each other");
    }
  }
}

}  // namespace

extern "C" {

void tk_default_options(tk_options* o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->blocks_per_cu = 1;
  o->fuse_pointwise = 1;
  o->fuse_epilogues = 1;
  o->inline_input_casts = 1;
  o->split_k_gemv = 1;
  o->threads_per_block = 256;
  o->fuse_updates = 1;
}

tk_status tk_compile(const char* ir, size_t ir_len, const tk_options* opts, int32_t device, tk_program** out) {
  if (!ir || !out) return fail(TK_E_ARG, "ir and out must not be NULL");
  *out = nullptr;
  TK_TRY({
    tk_options o;
    if (opts)
      o = *opts;
    else
      tk_default_options(&o);
    tk::Options so;
    if (o.blocks_per_cu < 1 || o.blocks_per_cu > 8) return fail(TK_E_ARG, "blocks_per_cu must be between 1 and 8");
    if (o.max_blocks < 0) return fail(TK_E_ARG, "max_blocks must be positive when provided");
    if (o.threads_per_block != 0 && o.threads_per_block != kBlock)
      return fail(TK_E_UNSUPPORTED, "threads_per_block must be 256 (four wave64) on gfx950");
    if (o.gemm_split_k != 0 && o.gemm_split_k != 1 && o.gemm_split_k != 2 && o.gemm_split_k != 4 && o.gemm_split_k != 8)
      return fail(TK_E_ARG, "gemm_split_k must be 0, 1, 2, 4 or 8");
    if (o.num_cus < 0) return fail(TK_E_ARG, "num_cus must not be negative");
    if (o.force_grid < 0) return fail(TK_E_ARG, "force_grid must not be negative");
    if (o.launch_mode != 0 && o.launch_mode != 1) return fail(TK_E_ARG, "launch_mode must be 0 or 1");
    if (o.gemm_tile < 0 || o.gemm_tile > 2) return fail(TK_E_ARG, "gemm_tile must be 0, 1 or 2");
    if (o.colsum_fusion < -1 || o.colsum_fusion > 1) return fail(TK_E_ARG, "colsum_fusion must be -1, 0 or 1");
    so.blocks_per_cu = o.blocks_per_cu;
    so.max_blocks = o.max_blocks;
    so.fuse_pointwise = o.fuse_pointwise != 0;
    so.fuse_epilogues = o.fuse_epilogues != 0;
    so.inline_input_casts = o.inline_input_casts != 0;
    so.split_k_gemv = o.split_k_gemv != 0;
    so.fuse_updates = o.fuse_updates != 0;
    so.barrier_every_op = o.barrier_every_op != 0;
    so.gemm_split_k = o.gemm_split_k;
    so.launch_mode = o.launch_mode;
    so.gemm_tile = o.gemm_tile;
    so.fast_epilogue = o.batch_epilogues == 0;
    so.colsum_fusion = o.colsum_fusion;
    so.num_cus = o.num_cus > 0 ? o.num_cus : 256;
    int occupancy = 0;
    hipFuncAttributes attr{};
    if (device >= 0) {
      hipDeviceProp_t prop;
      hipError_t e = hipGetDeviceProperties(&prop, device);
      if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
      if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(TK_E_DEVICE, std::string("an MI355X (gfx950) device is required, found ") + prop.gcnArchName);
      if (!prop.cooperativeLaunch) return fail(TK_E_DEVICE, "device does not support cooperative launch");
      so.num_cus = prop.multiProcessorCount;
    } else if (device != -1) {
      return fail(TK_E_ARG, "device must be >= 0, or -1 for a plan-only compile");
    }
    tk::Program prog = tk::parse_program(std::string(ir, ir_len));
    tk::validate_program(prog);
    auto* p = new tk_program();
    p->opts = so;
    p->device = device;
    try {
      p->plan = tk::schedule_program(prog, so);
    } catch (...) {
      delete p;
      throw;
    }
    int bpc = so.blocks_per_cu;
    if (device >= 0) {
      int cur = 0;
      hipGetDevice(&cur);
      hipSetDevice(device);
      hipError_t e = tk_device_occupancy(&occupancy);
      if (e == hipSuccess) e = tk_device_attributes(&attr);
      if (e == hipSuccess && occupancy < 1) {
        hipSetDevice(cur);
        delete p;
        return fail(TK_E_DEVICE, "kernel has no resident workgroups");
      }
      if (e == hipSuccess) e = hipMalloc(&p->d_plan, p->plan.bytes.size());
      if (e == hipSuccess) e = hipMemcpy(p->d_plan, p->plan.bytes.data(), p->plan.bytes.size(), hipMemcpyHostToDevice);
      void* hflag = nullptr;
      if (e == hipSuccess) e = hipHostMalloc(&hflag, 64, hipHostMallocMapped | hipHostMallocCoherent);
      if (e == hipSuccess) {
        p->h_abort = (volatile uint32_t*)hflag;
        p->h_abort[0] = p->h_abort[1] = 0u;
        void* dflag = nullptr;
        e = hipHostGetDevicePointer(&dflag, hflag, 0);
        p->d_abort = (uint32_t*)dflag;
      }
      hipSetDevice(cur);
      if (e != hipSuccess) {
        if (p->d_plan) hipFree(p->d_plan);
        if (p->h_abort) hipHostFree((void*)p->h_abort);
        delete p;
        return hip_fail(e, "plan upload");
      }
      bpc = std::min(bpc, occupancy);
    }
    long grid = (long)so.num_cus * bpc;
    if (o.force_grid > 0) {
      grid = std::min<long>(grid, o.force_grid);
    } else {
      grid = std::min<long>(grid, std::max(1, p->plan.max_items));
      if (so.max_blocks > 0) grid = std::min<long>(grid, so.max_blocks);
    }
    grid = std::min<long>(grid, (long)kMaxGrid);
    p->grid = (int)std::max<long>(1, grid);
    tk_stats& s = p->plan.stats;
    s.grid_size = p->grid;
    s.num_cus = so.num_cus;
    s.blocks_per_cu = bpc;
    s.occupancy = occupancy;
    s.vgprs = attr.numRegs;
    s.lds_bytes = (int32_t)attr.sharedSizeBytes;
    s.scratch_bytes = (int32_t)attr.localSizeBytes;
    *out = p;
    return TK_OK;
  })
}

tk_status tk_query(const tk_program* p, tk_stats* out) {
  if (!p || !out) return fail(TK_E_ARG, "program and out must not be NULL");
  *out = p->plan.stats;
  return TK_OK;
}

tk_status tk_dump_plan(const tk_program* p, char* buf, size_t len, size_t* needed) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  const std::string& d = p->plan.dump;
  if (needed) *needed = d.size() + 1;
  if (buf && len) {
    size_t n = std::min(len - 1, d.size());
    std::memcpy(buf, d.data(), n);
    buf[n] = 0;
  }
  return TK_OK;
}

tk_status tk_plan_bytes(const tk_program* p, void* buf, size_t len, size_t* needed) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  const auto& b = p->plan.bytes;
  if (needed) *needed = b.size();
  if (buf && len) std::memcpy(buf, b.data(), std::min(len, b.size()));
  return TK_OK;
}

tk_status tk_validate_into(const tk_program* p, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                           size_t n_out, const tk_tensor* workspace) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  TK_TRY({
    int device = p->device >= 0 ? p->device : (workspace ? workspace->device : 0);
    check_buffers(p, inputs, n_in, outputs, n_out, workspace, device);
    return TK_OK;
  })
}

tk_status tk_workspace_init(const tk_program* p, const tk_tensor* ws, void* stream) {
  if (!p || !ws) return fail(TK_E_ARG, "program and workspace must not be NULL");
  if (p->device < 0) return fail(TK_E_DEVICE, "plan-only program: no device");
  if (!ws->data || ws->ndim != 1 || (uint64_t)ws->shape[0] * tk::dtype_size((uint8_t)ws->dtype) < kHeaderBytes)
    return fail(TK_E_WORKSPACE, "workspace too small for its header");
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(p->device);
  hipError_t e = tk_device_zero_header((uint8_t*)ws->data, (hipStream_t)stream);
  hipSetDevice(cur);
  if (e != hipSuccess) return hip_fail(e, "workspace header init");
  if (p->h_abort) p->h_abort[0] = p->h_abort[1] = 0u;
  return TK_OK;
}

tk_status tk_allocate(const tk_program* p, const tk_tensor* inputs, size_t n_in, tk_alloc_fn alloc, void* ctx,
                      tk_tensor* outputs, size_t n_out, tk_tensor* workspace, void* stream) {
  if (!p || !alloc || !workspace) return fail(TK_E_ARG, "program, allocator and workspace must not be NULL");
  if (p->device < 0) return fail(TK_E_DEVICE, "plan-only program: no device");
  TK_TRY({
    const auto& pl = p->plan;
    check_inputs(p, inputs, n_in, p->device);
    if (n_out != pl.outputs.size()) return fail(TK_E_COUNT, "incorrect output buffer count");
    for (size_t s = 0; s < n_out; ++s) {
      tk_tensor& t = outputs[s];
      auto it = pl.inplace.find((int)s);
      if (it != pl.inplace.end()) {
        t = inputs[it->second];
        continue;
      }
      const tk::Spec& sp = pl.outputs[s];
      std::memset(&t, 0, sizeof(t));
      t.dtype = sp.dtype;
      t.ndim = (int32_t)sp.shape.size();
      int64_t acc = 1;
      for (int d = t.ndim - 1; d >= 0; --d) {
        t.shape[d] = sp.shape[d];
        t.strides[d] = acc;
        acc *= sp.shape[d];
      }
      uint64_t bytes = (uint64_t)acc * tk::dtype_size(sp.dtype);
      t.data = alloc(ctx, bytes, p->device);
      if (!t.data && bytes) return fail(TK_E_ARG, "allocator returned NULL for an output");
      t.storage_base = t.data;
      t.storage_bytes = bytes;
      t.device = p->device;
    }
    std::memset(workspace, 0, sizeof(*workspace));
    workspace->dtype = TK_I8;
    workspace->ndim = 1;
    workspace->shape[0] = (int64_t)pl.workspace_bytes;
    workspace->strides[0] = 1;
    workspace->data = alloc(ctx, pl.workspace_bytes, p->device);
    if (!workspace->data) return fail(TK_E_ARG, "allocator returned NULL for the workspace");
    workspace->storage_base = workspace->data;
    workspace->storage_bytes = pl.workspace_bytes;
    workspace->device = p->device;
    tk_status s = tk_workspace_init(p, workspace, stream);
    if (s != TK_OK) return s;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return TK_OK;
  })
}

namespace {

// Launch the step on checked buffers (tk_run_into, tk_run_into_noalloc).
tk_status launch_step(const tk_program* p, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                      size_t n_out, void* ws, void* stream, bool reset_header) {
  KArgs ka;
  std::memset(&ka, 0, sizeof(ka));
  ka.plan = (const uint8_t*)p->d_plan;
  ka.ws = (uint8_t*)ws;
  ka.deadline_ticks = p->deadline;
  ka.flags = p->dbg_flags;
  ka.stagger_seed = p->stagger;
  ka.host_abort = p->d_abort;
  const auto& pl = p->plan;
  ka.n_bases = (uint32_t)(pl.ws_base + 1);
  for (size_t i = 0; i < n_in; ++i) ka.bases[i] = inputs[i].data;
  for (size_t s = 0; s < n_out; ++s) ka.bases[pl.n_in + s] = outputs[s].data;
  ka.bases[pl.ws_base] = ws;
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != p->device) hipSetDevice(p->device);
  hipError_t e = hipSuccess;
  if (reset_header) e = tk_device_zero_header((uint8_t*)ws, (hipStream_t)stream);
  if (e == hipSuccess)
    e = p->opts.launch_mode == 1 ? tk_device_launch_resident(ka, p->grid, (hipStream_t)stream)
                                 : tk_device_launch(ka, p->grid, (hipStream_t)stream);
  if (cur != p->device) hipSetDevice(cur);
  if (e != hipSuccess) return hip_fail(e, p->opts.launch_mode == 1 ? "launch" : "cooperative launch");
  return TK_OK;
}

tk_status aborted_status(const tk_program* p) {
  return fail(TK_E_ABORTED, "a launch of this program stopped at a grid barrier that timed out (stage " +
                                std::to_string(p->h_abort[1]) +
                                "); its outputs are incomplete; re-initialise the workspace (tk_workspace_init) "
                                "before running again");
}

}  // namespace

tk_status tk_run_into(const tk_program* p, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                      size_t n_out, const tk_tensor* workspace, void* stream) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  if (p->device < 0) return fail(TK_E_DEVICE, "plan-only program: compile for a device to run");
  if (p->h_abort && p->h_abort[0] != 0u) return aborted_status(p);
  TK_TRY({
    check_buffers(p, inputs, n_in, outputs, n_out, workspace, p->device);
    return launch_step(p, inputs, n_in, outputs, n_out, workspace->data, stream, false);
  })
}

tk_status tk_run_into_noalloc(const tk_program* p, const tk_tensor* inputs, size_t n_in, const tk_tensor* outputs,
                              size_t n_out, void* stream) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  if (p->plan.workspace_bytes > kStaticWorkspaceBytes)
    return fail(TK_E_WORKSPACE, "the program needs a workspace of " + std::to_string(p->plan.workspace_bytes) +
                                    " bytes; the library's static workspace holds " +
                                    std::to_string(kStaticWorkspaceBytes) + " (use tk_run_into)");
  if (p->device < 0) return fail(TK_E_DEVICE, "plan-only program: compile for a device to run");
  if (p->h_abort && p->h_abort[0] != 0u) {
    // reported once: every call re-initialises the static workspace's header
    const tk_status st = aborted_status(p);
    p->h_abort[0] = p->h_abort[1] = 0u;
    return st;
  }
  TK_TRY({
    void* ws = nullptr;
    hipError_t e = tk_device_static_workspace(p->device, &ws);
    if (e != hipSuccess) return hip_fail(e, "static workspace lookup");
    tk_tensor w;
    std::memset(&w, 0, sizeof(w));
    w.data = ws;
    w.dtype = TK_I8;
    w.ndim = 1;
    w.shape[0] = (int64_t)kStaticWorkspaceBytes;
    w.strides[0] = 1;
    w.storage_base = ws;
    w.storage_bytes = kStaticWorkspaceBytes;
    w.device = p->device;
    check_buffers(p, inputs, n_in, outputs, n_out, &w, p->device);
    return launch_step(p, inputs, n_in, outputs, n_out, ws, stream, true);
  })
}

tk_status tk_workspace_status(const tk_tensor* ws, void* stream, int32_t* aborted, int32_t* stage) {
  if (!ws || !ws->data) return fail(TK_E_ARG, "workspace is NULL");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t a = 0, s = 0;
  e = hipMemcpy(&a, (uint8_t*)ws->data + kHdrAbort, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(&s, (uint8_t*)ws->data + kHdrAbortStage, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "workspace header read");
  if (aborted) *aborted = (int32_t)a;
  if (stage) *stage = (int32_t)s;
  return TK_OK;
}

tk_status tk_set_debug(tk_program* p, int32_t timestamps, uint32_t stagger_seed, uint64_t deadline_ticks) {
  if (!p) return fail(TK_E_ARG, "program is NULL");
  p->dbg_flags = (timestamps ? K_TIMESTAMPS : 0u) | (stagger_seed ? K_STAGGER : 0u);
  p->stagger = stagger_seed;
  p->deadline = deadline_ticks;
  return TK_OK;
}

tk_status tk_read_timestamps(const tk_program* p, const tk_tensor* ws, void* stream, uint64_t* out, size_t n) {
  if (!p || !ws || !out) return fail(TK_E_ARG, "NULL argument");
  size_t want = std::min<size_t>(n, 4 * (size_t)std::min<int>(p->plan.n_stages, (int)kMaxTimedStages));
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpy(out, (uint8_t*)ws->data + kHdrStamps, want * 8, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "timestamp read");
  return TK_OK;
}

void tk_destroy(tk_program* p) {
  if (!p) return;
  if (p->d_plan) {
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(p->device);
    hipFree(p->d_plan);
    hipSetDevice(cur);
  }
  if (p->h_abort) hipHostFree((void*)p->h_abort);
  delete p;
}

const char* tk_last_error(void) { return g_err.c_str(); }

}  // extern "C"
