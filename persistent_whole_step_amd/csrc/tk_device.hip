// The persistent whole-step kernel for gfx950 (MI355X).
//
// One cooperative launch runs a whole compiled program: every workgroup walks
// the plan's stages, takes the stage's work items round-robin
// (item = blockIdx.x + i * gridDim.x), and all workgroups meet at a
// global-memory grid barrier between stages.  This is the execution model of
// the trainkernel generator (trainkernel wheel, codegen.py: operators emitted
// in topological order with a grid sync between dependent ones, and the device
// helpers of its CUDA preamble), re-designed as an interpreter of a
// device-resident plan:
//   * pointwise work and every epilogue run on one expression machine that is
//     compiled into the kernel exactly once; each task kind feeds it batches of
//     16 elements per thread (two 8-wide chunks, or sixteen single elements)
//     through LDS, so the code every stage runs stays small;
//   * contractions with bf16/f16 operands run on MFMA 32x32x16 tiles with
//     LDS double buffering; other dtypes use an fp32-FMA tile whose per-output
//     accumulation is sequential in k;
//   * one-row int8-weight products stream the weight once, split along K over
//     the 64 lanes of a wave;
//   * reductions sum fixed partitions in a fixed order (deterministic, every
//     element covered).
// Every pointer into device memory carries the global address space and every
// LDS access the local one, so a wait for LDS never waits for global traffic
// (generic "flat" accesses count against both wait counters).
// Built with -ffp-contract=off: no implicit fused multiply-adds, so pointwise
// results equal IEEE binary32 step by step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "plan.h"

using namespace tkplan;

#define DEV __device__ __forceinline__
#define GLOBAL __attribute__((address_space(1)))
#define LDS __attribute__((address_space(3)))

namespace {

// Workgroup LDS arena (128 KB).  A contraction's operand ring uses all of it
// during its main loop; afterwards the fp32 C tile (at most 128 x 132 floats)
// takes the bottom, and the expression machine's third slot and its exchange
// the top 48 KB.  Every other task uses the bottom 80 KB for staging or
// scratch.
constexpr int kSmemBytes = 81920;        // staging / scratch region below the slots
constexpr int kSlot2Off = kSmemBytes;    // machine slot 2
constexpr int kXvOff = kSmemBytes + 16384;  // machine exchange: values (slot 0)
constexpr int kXeOff = kSmemBytes + 32768;  // machine exchange: chunk starts (slot 1)
constexpr int kVmElems = 16;                       // elements per thread per machine batch

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Workgroup-shared storage.
__shared__ __attribute__((aligned(16))) uint8_t g_smem[kArenaBytes];  // see kArenaBytes
__shared__ __attribute__((aligned(16))) uint8_t g_plan[kPlanLds];    // current stage's descriptors
// Machine exchange (in the arena's top 32 KB): values [element][thread] and
// the first linear element of each chunk [chunk][thread].
DEV LDS float& xv(uint32_t tid, int j) { return ((LDS float*)(g_smem + kXvOff))[j * kBlock + tid]; }
DEV LDS uint32_t& xe(uint32_t tid, int q) { return ((LDS uint32_t*)(g_smem + kXeOff))[q * kBlock + tid]; }
// Slots of the expression machine live in LDS, laid out like the exchange
// (element j of thread t at j * kBlock + t, so each thread touches only its
// own words): slot 0 reuses the value exchange and slot 1 the index exchange
// (both are read at the start of a batch and rewritten only at its end),
// slot 2 has a region of its own below them.  Holding them in registers made
// every join of the interpreter loop copy them.
static_assert(kMaxSlots == 3, "three LDS slots");
DEV LDS float* slot_base(uint32_t k) {
  return (LDS float*)(g_smem + (k == 0 ? kXvOff : k == 1 ? kXeOff : kSlot2Off));
}
static_assert(kSlot2Off + kVmElems * kBlock * 4 == kXvOff, "arena layout");
static_assert(kXeOff + kVmElems * kBlock * 4 == (int)kArenaBytes, "arena layout");
static_assert(128 * 132 * 4 <= kSmemBytes, "the largest C tile fits below the slots");

// ------------------------------------------------------------ conversions --

DEV float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32; NaN stays
// NaN, subnormals kept).
DEV uint32_t f32_to_bf16_bits(float f) {
  const __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

DEV float f16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

DEV uint32_t f32_to_f16_bits(float f) {
  _Float16 v = (_Float16)f;  // v_cvt_f16_f32: round-to-nearest-even, subnormals kept
  return (uint32_t)__builtin_bit_cast(uint16_t, v);
}

DEV float half_bits_to_f32(uint32_t h, bool bf) { return bf ? bf16_bits_to_f32(h) : f16_bits_to_f32(h); }

// Eight 16-bit values (one 16-byte chunk) widened to fp32, the dtype fixed
// per call (no per-element dtype select); and fp32 values narrowed (RNE) and
// packed two to a word.
template <bool BF>
DEV void widen8(u32x4 v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (BF) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    } else {
      x[2 * j] = f16_bits_to_f32(v[j] & 0xffffu);
      x[2 * j + 1] = f16_bits_to_f32(v[j] >> 16);
    }
  }
}
template <bool BF>
DEV uint32_t narrow2(float lo, float hi) {
  return BF ? f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16) : f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
}
DEV uint32_t f32_to_half_bits(float f, bool bf) { return bf ? f32_to_bf16_bits(f) : f32_to_f16_bits(f); }

DEV uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DEV int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)(((uint64_t)uniform((uint32_t)(u >> 32)) << 32) | uniform((uint32_t)u));
}

template <class T>
DEV bool aligned16(const GLOBAL T* p) {
  return ((uintptr_t)p & 15) == 0;
}

// ------------------------------------------------------- launch context --
// The argument block is read once per launch: scalars into registers, the
// base-pointer table into LDS.  Later reads never go back to the kernel
// argument segment.
__shared__ uint64_t g_bases[kMaxBases];

struct Ctx {
  GLOBAL uint8_t* ws;          // workspace: header, then arena
  const GLOBAL uint8_t* plan;  // device-resident plan
  uint32_t flags;              // K_* debug switches
  uint32_t stagger_seed;
  uint32_t* host_abort;        // pinned host words [aborted, stage], or null
};

// Record a stopped launch: the workspace's abort word and stage, and the
// program's pinned host words that tk_run_into reads before the next launch.
DEV void set_abort(const Ctx& ka, uint32_t stage) {
  GLOBAL uint32_t* abort = (GLOBAL uint32_t*)(ka.ws + kHdrAbort);
  GLOBAL uint32_t* abort_stage = (GLOBAL uint32_t*)(ka.ws + kHdrAbortStage);
  __hip_atomic_store(abort_stage, stage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (ka.host_abort) {
    __hip_atomic_store(ka.host_abort + 1, stage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(ka.host_abort, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

DEV GLOBAL uint8_t* base_ptr(const Ctx&, uint32_t base) {
  return (GLOBAL uint8_t*)uniform64((int64_t)((const LDS uint64_t*)g_bases)[base]);
}
// ------------------------------------------------------- element access --

DEV GLOBAL float* ws_f32(const Ctx& ka, uint64_t off) { return (GLOBAL float*)(ka.ws + off); }

DEV float load_elem(const GLOBAL uint8_t* p, uint32_t dt, int64_t idx) {
  if (dt == DT_F32) return ((const GLOBAL float*)p)[idx];
  if (dt == DT_I8) return (float)((const GLOBAL int8_t*)p)[idx];
  return half_bits_to_f32(((const GLOBAL uint16_t*)p)[idx], dt == DT_BF16);
}

// Loads of all C chunks of one view operand, issued before any is used.
// vec (uniform): unit inner stride, 16-byte aligned base, and every chunk
// start 16-byte aligned, so each 8-wide chunk is one (bf16/f16) or two (f32)
// 16-byte loads.  Every index must address an element of the view (dead
// chunks point at its first element).
template <int W, int C>
DEV void load_chunks(const GLOBAL uint8_t* p, uint32_t dt, bool vec, int32_t s, const int32_t (&idx)[C],
                     float (&x)[C][W]) {
  if (dt == DT_F32) {
    const GLOBAL float* q = (const GLOBAL float*)p;
    if (W == 8 && vec) {
      u32x4 r[C][2];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        r[c][0] = *(const GLOBAL u32x4*)(q + idx[c]);
        r[c][1] = *(const GLOBAL u32x4*)(q + idx[c] + 4);
      }
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) x[c][j] = __uint_as_float(r[c][j / 4][j % 4]);
    } else if (W == 8 && s == 0) {
      float r[C];
#pragma unroll
      for (int c = 0; c < C; ++c) r[c] = q[idx[c]];
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) x[c][j] = r[c];
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) x[c][j] = q[idx[c] + j * s];
    }
  } else if (dt == DT_I8) {
    const GLOBAL int8_t* q = (const GLOBAL int8_t*)p;
    int32_t r[C][W];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < W; ++j) r[c][j] = q[idx[c] + j * s];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < W; ++j) x[c][j] = (float)r[c][j];
  } else {
    const GLOBAL uint16_t* q = (const GLOBAL uint16_t*)p;
    const bool bf = dt == DT_BF16;
    uint32_t h[C][W];
    if (W == 8 && vec) {
      u32x4 r[C];
#pragma unroll
      for (int c = 0; c < C; ++c) r[c] = *(const GLOBAL u32x4*)(q + idx[c]);
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) h[c][j] = (j & 1) ? r[c][j / 2] >> 16 : r[c][j / 2] & 0xffffu;
    } else if (W == 8 && s == 0) {
      uint32_t r[C];
#pragma unroll
      for (int c = 0; c < C; ++c) r[c] = q[idx[c]];
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) h[c][j] = r[c];
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int j = 0; j < W; ++j) h[c][j] = q[idx[c] + j * s];
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < W; ++j) x[c][j] = half_bits_to_f32(h[c][j], bf);
  }
}

// Stores of the live chunks (bit q of `live`), converted to the view's dtype.
template <int W, int C>
DEV void store_chunks(GLOBAL uint8_t* p, uint32_t dt, bool vec, int32_t s, const int32_t (&idx)[C], uint32_t live,
                      const float (&x)[C][W]) {
  if (dt == DT_F32) {
    GLOBAL float* q = (GLOBAL float*)p;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (!(live & (1u << c))) continue;
      if (W == 8 && vec) {
        u32x4 r0, r1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r0[j] = __float_as_uint(x[c][j]);
          r1[j] = __float_as_uint(x[c][4 + j]);
        }
        *(GLOBAL u32x4*)(q + idx[c]) = r0;
        *(GLOBAL u32x4*)(q + idx[c] + 4) = r1;
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) q[idx[c] + j * s] = x[c][j];
      }
    }
  } else if (dt != DT_I8) {
    GLOBAL uint16_t* q = (GLOBAL uint16_t*)p;
    const bool bf = dt == DT_BF16;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (!(live & (1u << c))) continue;
      uint32_t h[W];
#pragma unroll
      for (int j = 0; j < W; ++j) h[j] = f32_to_half_bits(x[c][j], bf);
      if (W == 8 && vec) {
        u32x4 r;
#pragma unroll
        for (int j = 0; j < W / 2; ++j) r[j] = h[2 * j] | (h[2 * j + 1] << 16);
        *(GLOBAL u32x4*)(q + idx[c]) = r;
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) q[idx[c] + j * s] = (uint16_t)h[j];
      }
    }
  }
}

// e / d for the divisor constants (m, l) the host computed for d.
DEV uint32_t udiv(uint32_t e, uint32_t m, uint32_t l) {
  const uint32_t t = __umulhi(m, e);
  const uint32_t sh1 = l ? 1u : 0u, sh2 = l ? l - 1u : 0u;
  return (t + ((e - t) >> sh1)) >> sh2;
}

// ------------------------------------------------------ debug trace --
// With K_TIMESTAMPS, lane 0 of workgroup 0 also records up to kTraceLen
// fine-grained timestamps of the current launch into the workspace header.
constexpr uint32_t kTraceOff = 14336;
constexpr uint32_t kTraceLen = 64;

DEV void trace_stamp(const Ctx& ka, uint32_t tag) {
  if (!(ka.flags & K_TIMESTAMPS) || blockIdx.x != 0 || threadIdx.x != 0) return;
  __shared__ uint32_t s_trace_n;  // entries written by this launch (reset at launch start)
  if (tag == 0xffffffffu) {
    s_trace_n = 0;
    return;
  }
  const uint32_t i = s_trace_n;
  if (i >= kTraceLen) return;
  GLOBAL uint64_t* ent = (GLOBAL uint64_t*)(ka.ws + kTraceOff + 8) + 2 * i;
  ent[0] = tag;
  ent[1] = __builtin_amdgcn_s_memrealtime();
  s_trace_n = i + 1;
  *(GLOBAL uint32_t*)(ka.ws + kTraceOff) = i + 1;
}

// ------------------------------------------------------ plan access (LDS) --

// A task's descriptor with every word made wave-uniform (scalar registers).
DEV DTask load_task(uint32_t i) {
  constexpr int N = sizeof(DTask) / 4;
  static_assert(sizeof(DTask) % 4 == 0, "DTask words");
  const LDS uint32_t* w = (const LDS uint32_t*)(g_plan + i * sizeof(DTask));
  struct Words {
    uint32_t u[N];
  } r;
#pragma unroll
  for (int k = 0; k < N; ++k) r.u[k] = uniform(w[k]);
  return __builtin_bit_cast(DTask, r);
}

DEV uint32_t task_item_begin(uint32_t i) {
  return uniform(((const LDS DTask*)g_plan)[i].item_begin);
}

// A view with 32-bit offset and strides (the compiler rejects programs whose
// views or workspace address 2^31 elements or more), in scalar registers.
struct VView {
  int32_t offset;
  int32_t stride[kMaxDims];
  uint32_t base;
  uint32_t dtype;
};

DEV VView load_view(uint32_t off) {
  const LDS DView& v = *(const LDS DView*)(g_plan + off);
  VView r;
  r.offset = (int32_t)uniform((uint32_t)v.offset);
#pragma unroll
  for (int d = 0; d < kMaxDims; ++d) r.stride[d] = (int32_t)uniform((uint32_t)v.stride[d]);
  r.base = uniform(v.base);
  r.dtype = uniform(v.dtype);
  return r;
}

// Element index of a view at coordinates c (dims past the task's rank have
// coordinate 0 and stride 0).
DEV int32_t view_index(const VView& v, const uint32_t (&c)[kMaxDims]) {
  int32_t idx = v.offset;
#pragma unroll
  for (int d = 0; d < kMaxDims; ++d) idx += (int32_t)c[d] * v.stride[d];
  return idx;
}

// The stride of the innermost iteration dim.  Written as a chain of
// selects on scalars: the compiler must not turn it into an indexed load from
// a stack copy of the strides (private memory).
DEV int32_t inner_stride(const VView& v, uint32_t nd) {
  int32_t s = v.stride[0];
  s = nd >= 2 ? v.stride[1] : s;
  asm volatile("" : "+s"(s));
  s = nd >= 3 ? v.stride[2] : s;
  asm volatile("" : "+s"(s));
  s = nd >= 4 ? v.stride[3] : s;
  return s;
}

// ------------------------------------------------------ expression machine --

// One batch for the machine: a program over an iteration space.
struct Batch {
  uint32_t ins;         // byte offset (in the LDS plan) of the first instruction
  uint32_t n;           // instructions
  uint32_t width;       // 8: two 8-wide chunks per thread; 1: sixteen single elements
  uint32_t nd;
  uint32_t dims[kMaxDims];
  uint32_t dmul[kMaxDims], dsh[kMaxDims];  // division constants for dims[1..nd-1]
  uint32_t accumulate;  // reductions: add the results into the thread's sums
};

// Coordinates of linear element e of the batch's iteration space (row-major).
DEV void unravel(uint32_t e, const Batch& b, uint32_t (&c)[kMaxDims]) {
#pragma unroll
  for (int d = kMaxDims - 1; d >= 1; --d) {
    if ((uint32_t)d < b.nd) {
      const uint32_t q = udiv(e, b.dmul[d], b.dsh[d]);
      c[d] = e - q * b.dims[d];
      e = q;
    } else {
      c[d] = 0;
    }
  }
  c[0] = e;
}

// Run a program on C chunks of W elements (C * W == 16).  Chunk q starts at
// linear element xe(tid, q) of the iteration space and covers W consecutive
// elements along its last dim; chunks whose bit in `live` is clear touch no
// memory.  The accumulators start from and end in the exchange values.  The
// loads of all chunks of one instruction are issued before any is used, so an
// instruction costs one memory latency, not one per element.
template <int W, int C>
DEV void vm_run(uint32_t tid, const Ctx& ka, const Batch& b, uint32_t views_off, uint32_t live) {
  float acc[C][W];
  uint32_t c[C][kMaxDims];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    unravel(xe(tid, q), b, c[q]);
#pragma unroll
    for (int j = 0; j < W; ++j) acc[q][j] = xv(tid, q * W + j);
  }
  for (uint32_t pc = 0; pc < b.n; ++pc) {
    const LDS uint32_t* iw = (const LDS uint32_t*)(g_plan + b.ins + pc * sizeof(DIns));
    const uint32_t w0 = uniform(iw[0]), w1 = uniform(iw[1]);
    const float a = __uint_as_float(uniform(iw[2])), sv = __uint_as_float(uniform(iw[3]));
    const uint32_t op = w0 & 0xff, src = (w0 >> 8) & 0xff, rnd = (w0 >> 16) & 0xff, rev = w0 >> 24;
    const uint32_t arg = w1 & 0xffff;
    float x[C][W];
    if (src == SRC_VIEW || op == VM_STORE) {
      const VView v = load_view(views_off + arg * sizeof(DView));
      const int32_t s = inner_stride(v, b.nd);
      const uint32_t dt = v.dtype;
      GLOBAL uint8_t* p = base_ptr(ka, v.base);
      // 16-byte chunk accesses: unit inner stride, aligned base, and offset and
      // outer strides multiples of the elements per 16 bytes (chunk starts lie
      // at multiples of 8 along the inner dim)
      const int32_t epc = dt == DT_F32 ? 4 : 8;
      bool vec = W == 8 && s == 1 && dt != DT_I8 && ((uintptr_t)p & 15) == 0 && v.offset % epc == 0;
#pragma unroll
      for (int d = 0; d + 1 < kMaxDims; ++d)
        if ((uint32_t)d + 1 < b.nd) vec = vec && v.stride[d] % epc == 0;
      int32_t idx[C];
#pragma unroll
      for (int q = 0; q < C; ++q) idx[q] = view_index(v, c[q]);
      if (op == VM_STORE) {
        store_chunks<W, C>(p, dt, vec, s, idx, live, acc);
        continue;
      }
      load_chunks<W, C>(p, dt, vec, s, idx, x);
      // Wait for the operand here, on the only path that loads one: the
      // compiler would otherwise wait at its use on every path, and that wait
      // would also cover stores of earlier instructions still in flight.
      __builtin_amdgcn_s_waitcnt(0);
    } else if (src == SRC_SLOT) {
      const LDS float* sb = slot_base(arg);
#pragma unroll
      for (int q = 0; q < C; ++q)
#pragma unroll
        for (int j = 0; j < W; ++j) x[q][j] = sb[(q * W + j) * kBlock + tid];
    } else {
      const float k = src == SRC_SCALAR ? sv : 0.0f;
#pragma unroll
      for (int q = 0; q < C; ++q)
#pragma unroll
        for (int j = 0; j < W; ++j) x[q][j] = k;
    }
#define TK_EACH(expr)                             \
  _Pragma("unroll") for (int q = 0; q < C; ++q)   \
  _Pragma("unroll") for (int j = 0; j < W; ++j) { \
    float& y = acc[q][j];                         \
    const float o = x[q][j];                      \
    (void)o;                                      \
    expr;                                         \
  }
    switch (op) {
      case VM_LOAD: TK_EACH(y = o) break;
      case VM_ADD:
        if (rev) { TK_EACH(float t = a * y; y = o + t) }
        else { TK_EACH(float t = a * o; y = y + t) }
        break;
      case VM_SUB:
        if (rev) { TK_EACH(float t = a * y; y = o - t) }
        else { TK_EACH(float t = a * o; y = y - t) }
        break;
      case VM_MUL: TK_EACH(y = y * o) break;
      case VM_DIV:
        if (rev) { TK_EACH(y = o / y) }
        else { TK_EACH(y = y / o) }
        break;
      case VM_NEG: TK_EACH(y = -y) break;
      case VM_RELU: TK_EACH(y = y < 0.0f ? 0.0f : y) break;
      case VM_SQUARE: TK_EACH(y = y * y) break;
      case VM_POW: TK_EACH(y = powf(y, a)) break;
      case VM_TB:
        if (rev) { TK_EACH(y = y <= a ? 0.0f : o) }
        else { TK_EACH(y = o <= a ? 0.0f : y) }
        break;
      case VM_SAVE: {
        LDS float* sb = slot_base(arg);
        TK_EACH(sb[(q * W + j) * kBlock + tid] = y)
        break;
      }
      case VM_SCALE: TK_EACH(y = a * y) break;
      case VM_ZERO: TK_EACH(y = 0.0f) break;
      case VM_SQRT: TK_EACH(y = sqrtf(y)) break;
      default: break;
    }
#undef TK_EACH
    if (rnd == DT_BF16) {
#pragma unroll
      for (int q = 0; q < C; ++q)
#pragma unroll
        for (int j = 0; j < W; ++j) acc[q][j] = bf16_bits_to_f32(f32_to_bf16_bits(acc[q][j]));
    } else if (rnd == DT_F16) {
#pragma unroll
      for (int q = 0; q < C; ++q)
#pragma unroll
        for (int j = 0; j < W; ++j) acc[q][j] = f16_bits_to_f32(f32_to_f16_bits(acc[q][j]));
    }
  }
#pragma unroll
  for (int q = 0; q < C; ++q)
#pragma unroll
    for (int j = 0; j < W; ++j) xv(tid, q * W + j) = acc[q][j];
}

// ------------------------------------------------------------ work items --
// Every work item runs as: an optional prologue (a contraction's main loop,
// a GEMV's dot products), then batches b = 0, 1, ... each filled by the task
// kind, run on the machine and consumed by the task kind, until the kind
// reports no further batch.  Batch decisions are uniform across the workgroup.

// Per-item state carried across batches.
struct ItemState {
  uint32_t m0, n0, split_index;  // contraction tile origin / split-K part
  int bm, bn;                    // contraction tile size
  float acc;                     // reductions: this thread's running sum
  float acc8[8];
};

// Tile index for work item `local` of a contraction: the eight XCDs take
// workgroups round-robin, so items with equal local % 8 share an XCD; give
// each such class a contiguous run of tiles (row-major), which share operand
// panels in that XCD's L2.
DEV uint32_t xcd_tile(uint32_t local, uint32_t tiles) {
  if (tiles % 8 != 0) return local;
  return (local % 8) * (tiles / 8) + local / 8;
}

// Tile coordinates of tile-order index `tile`: group-major, group_m tile rows
// per group, column by column within a group (group_m divides tiles_m), so a
// run of consecutive indices covers a compact block of the output.
DEV void tile_coords(const DTask& t, uint32_t tile, uint32_t& tm, uint32_t& tn) {
  const uint32_t gm = t.group_m > 1 ? t.group_m : 1;
  const uint32_t gsz = gm * t.tiles_n;
  const uint32_t g = tile / gsz, r = tile % gsz;
  tm = g * gm + r % gm;
  tn = r / gm;
}

// ------------------------------------------------------ fp32-FMA contraction --
// 64x64 output tile, 256 threads, each thread a 4x4 block; K staged 32 deep in
// a double-buffered LDS ring, the next slice's loads issued before the current
// slice is consumed.  Each output accumulates acc = fma(a_k, b_k, acc) for
// k = 0, 1, ... in order.

// The 8 elements of one thread, all loads issued before any is used: the
// operand dtype is a template parameter, so no branch separates the loads.
template <uint32_t DT>
DEV void simt_load_t(uint32_t tid, const GLOBAL uint8_t* p, const VView& v, bool mn_contig, bool is_a, uint32_t r0,
                     uint32_t rmax, uint32_t k0, uint32_t kmax, float (&reg)[8]) {
  const int64_t s_r = is_a ? v.stride[0] : v.stride[1], s_k = is_a ? v.stride[1] : v.stride[0];
  int64_t idx[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + i * kBlock;  // 0 .. 2047 over a 64 x 32 slice
    const int r = mn_contig ? q % 64 : q / 32, kk = mn_contig ? q / 64 : q % 32;
    const uint32_t gr = r0 + r, gk = k0 + kk;
    ok[i] = gr < rmax && gk < kmax;
    idx[i] = v.offset + (int64_t)(ok[i] ? gr : 0) * s_r + (int64_t)(ok[i] ? gk : 0) * s_k;
  }
  float x[8];
  if constexpr (DT == DT_F32) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ((const GLOBAL float*)p)[idx[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = w[i];
  } else if constexpr (DT == DT_I8) {
    int32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ((const GLOBAL int8_t*)p)[idx[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)w[i];
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ((const GLOBAL uint16_t*)p)[idx[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = half_bits_to_f32(w[i], DT == DT_BF16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) reg[i] = ok[i] ? x[i] : 0.0f;
}

DEV void simt_load(uint32_t tid, const GLOBAL uint8_t* p, const VView& v, bool mn_contig, bool is_a, uint32_t r0,
                   uint32_t rmax, uint32_t k0, uint32_t kmax, float (&reg)[8]) {
  switch (v.dtype) {
    case DT_F32: simt_load_t<DT_F32>(tid, p, v, mn_contig, is_a, r0, rmax, k0, kmax, reg); break;
    case DT_BF16: simt_load_t<DT_BF16>(tid, p, v, mn_contig, is_a, r0, rmax, k0, kmax, reg); break;
    case DT_F16: simt_load_t<DT_F16>(tid, p, v, mn_contig, is_a, r0, rmax, k0, kmax, reg); break;
    default: simt_load_t<DT_I8>(tid, p, v, mn_contig, is_a, r0, rmax, k0, kmax, reg); break;
  }
}

DEV void simt_store(uint32_t tid, LDS float* s, bool mn_contig, const float (&reg)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + i * kBlock;
    const int r = mn_contig ? q % 64 : q / 32, kk = mn_contig ? q / 64 : q % 32;
    s[kk * 68 + r] = reg[i];
  }
}

DEV void gemm_simt(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t item, ItemState& st) {
  const uint32_t tile = xcd_tile(item, t.tiles_m * t.tiles_n);
  uint32_t tm, tn;
  tile_coords(t, tile, tm, tn);
  const uint32_t m0 = tm * 64, n0 = tn * 64;
  LDS float* As0 = (LDS float*)g_smem;
  LDS float* As1 = As0 + 32 * 68;
  LDS float* Bs0 = As0 + 2 * 32 * 68;
  LDS float* Bs1 = As0 + 3 * 32 * 68;
  const VView A = load_view(views_off + t.va * sizeof(DView)), B = load_view(views_off + t.vb * sizeof(DView));
  const GLOBAL uint8_t* pa = base_ptr(ka, A.base);
  const GLOBAL uint8_t* pb = base_ptr(ka, B.base);
  const bool a_mc = A.stride[0] == 1 && A.stride[1] != 1;  // A unit-stride along m
  const bool b_nc = B.stride[1] == 1;                      // B unit-stride along n
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  const uint32_t nk = (t.k + 31) / 32;
  float ra[8], rb[8];
  if (nk > 0) {
    simt_load(tid, pa, A, a_mc, true, m0, t.m, 0, t.k, ra);
    simt_load(tid, pb, B, b_nc, false, n0, t.n, 0, t.k, rb);
    simt_store(tid, As0, a_mc, ra);
    simt_store(tid, Bs0, b_nc, rb);
  }
  __syncthreads();
  for (uint32_t kt = 0; kt < nk; ++kt) {
    const bool odd = kt & 1;
    if (kt + 1 < nk) {
      simt_load(tid, pa, A, a_mc, true, m0, t.m, (kt + 1) * 32, t.k, ra);
      simt_load(tid, pb, B, b_nc, false, n0, t.n, (kt + 1) * 32, t.k, rb);
    }
    const LDS float* as = odd ? As1 : As0;
    const LDS float* bs = odd ? Bs1 : Bs0;
    const uint32_t kend = t.k - kt * 32 < 32 ? t.k - kt * 32 : 32;
    for (uint32_t kk = 0; kk < kend; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk * 68 + ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = bs[kk * 68 + tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      simt_store(tid, odd ? As0 : As1, a_mc, ra);
      simt_store(tid, odd ? Bs0 : Bs1, b_nc, rb);
    }
    __syncthreads();
  }
  LDS float* C = (LDS float*)g_smem;  // [64][68]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) C[(ty * 4 + i) * 68 + tx * 4 + j] = acc[i][j];
  st.m0 = m0;
  st.n0 = n0;
  st.bm = 64;
  st.bn = 64;
  st.split_index = 0;
}

// ------------------------------------------------------- MFMA contraction --
// Tile BM x BN, K staged 64 deep; 4 waves in a 2x2 grid, each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA accumulators.
//
// Fast path (interior tile, whole 64-deep slices, 16-byte aligned rows):
// operands go from global memory straight into LDS (global_load_lds, 16
// bytes per lane; each wave instruction fills one contiguous 1 KB block, the
// lane's source address choosing what lands where), in a ring of S stages
// with S - 1 slices in flight.  An operand with unit stride along k is staged
// as [row][64 k] (128-byte rows, 16-byte chunk c of row r at position
// c ^ ((r ^ r>>3) & 7)) and read with 16-byte fragment loads.  An operand
// with unit stride along M/N is staged as it lies, [k][rows] (chunk c of k-row
// k at c ^ kswz(k)), and read with ds_read_b64_tr_b16: lane i of each 16-lane
// group addresses k-row kbase + i/4, columns nbase + 4(i%4), and receives the
// four k values of column nbase + (its lane within the group), so two reads
// give the 8 k values of an MFMA fragment.  Both swizzles keep every access
// pattern at most two-way per bank.  Other tiles stage element by element in
// the k-major layout.

constexpr int kBK = 64;
constexpr int kPitch = kBK;  // halfs per k-major staged row

// Element offset (in halfs) of (row, 16-byte chunk c) in a k-major operand.
DEV int swz(int row, int c) { return row * kPitch + ((c ^ ((row ^ (row >> 3)) & 7)) << 3); }

// Chunk position swizzle of k-row k in a row-major ([k][R]) operand.
template <int R>
DEV int kswz(int k) {
  if (R == 128) return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1);
  return (((k >> 1) & 1) << 2) ^ (((k >> 3) & 1) << 1);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct-to-LDS staging of one operand: R tile rows x 64 k per slice, R/8 KB,
// R/32 blocks of 1 KB per wave.
template <int R>
struct DirectOp {
  static constexpr int NB = R / 32;
  const GLOBAL uint8_t* src[NB];  // this lane's source for slice 0, per block
  int64_t kstep;                  // bytes from one slice to the next
  uint32_t wave;
  DEV void init(uint32_t tid, bool kc, const GLOBAL uint16_t* q, int64_t off, int64_t sr, int64_t sk, uint32_t r0,
                uint32_t k0) {
    wave = uniform(tid / 64);  // the LDS destination (M0) must be wave-uniform
    const int lane = tid % 64;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = (int)wave + 4 * i;  // block index
      if (kc) {
        // block b: rows 8b .. 8b+7; lane -> (row, position); load the chunk the swizzle puts there
        const int r = 8 * b + lane / 8, p = lane % 8;
        const int c = p ^ ((r ^ (r >> 3)) & 7);
        src[i] = (const GLOBAL uint8_t*)(q + off + (int64_t)(r0 + r) * sr + k0 + c * 8);
      } else {
        // block b: k-rows b*(512/R) ..; R/8 chunks per k-row
        constexpr int cpr = R / 8;
        const int k = b * (512 / R) + lane / cpr, p = lane % cpr;
        const int c = p ^ kswz<R>(k);
        src[i] = (const GLOBAL uint8_t*)(q + off + (int64_t)(k0 + k) * sk + r0 + c * 8);
      }
    }
    kstep = kc ? (int64_t)kBK * 2 : (int64_t)kBK * sk * 2;
  }
  // Issue the loads of `slice` into the operand region at LDS byte offset `lds`.
  // Written as inline asm so the compiler does not order every later LDS read
  // behind these writes (it cannot tell the ring stages apart); the main loop
  // waits for them explicitly (vmcnt) and with a workgroup barrier.
  DEV void issue(uint32_t slice, uint32_t lds) const {
    const uint32_t base = (uint32_t)(uintptr_t)(LDS uint8_t*)g_smem + lds + wave * 1024;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const GLOBAL uint8_t* g = src[i] + (int64_t)slice * kstep;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base + 4096 * i) : "m0");
    }
  }
};

// General operand path: element by element into the k-major layout, zero outside.
template <int R>
DEV void slow_stage(uint32_t tid, const GLOBAL uint16_t* q, int64_t off, int64_t sr, int64_t sk, uint32_t r0,
                    uint32_t rmax, uint32_t k0, uint32_t kmax, LDS uint16_t* lds) {
  // consecutive threads walk the operand's unit-stride dimension when it has one
  const bool kfast = sk == 1 || sr != 1;
  for (int p = tid; p < R * kBK; p += kBlock) {
    const int r = kfast ? p / kBK : p % R, kk = kfast ? p % kBK : p / R;
    const uint32_t gr = r0 + r, gk = k0 + kk;
    const bool ok = gr < rmax && gk < kmax;
    const uint16_t v = q[off + (int64_t)(ok ? gr : 0) * sr + (int64_t)(ok ? gk : 0) * sk];
    lds[swz(r, kk / 8) + kk % 8] = ok ? v : (uint16_t)0;
  }
}

template <bool BF16>
DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// s plus the eight 16-bit values of a fragment, as dot products with (1, 1)
// (the products are exact; each step rounds once to fp32).
template <bool BF16>
DEV float frag_sum(u32x4 v, float s) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // (a bit cast of the subscript v[q] itself reads element 0: copy it out)
    const uint32_t w = v[q];
    if (BF16)
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u), s,
                                          false);
    else
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3c003c00u), s, false);
  }
  return s;
}

// MFMA fragment of `row0 + lane%32` (rows of an R-row operand), k = kk + 8*(lane/32) .. +7.
// KM: the operand is staged k-major (else row-major, read transposed).
template <int R, bool KM>
DEV u32x4 frag(uint32_t tid, const LDS uint16_t* s, int row0, int kk) {
  const int lane = tid % 64;
  if (KM) return *(const LDS u32x4*)(s + swz(row0 + lane % 32, kk / 8 + lane / 32));
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int g = lane / 16, i = lane % 16;
  const int n = row0 + 16 * (g % 2) + 4 * (i % 4);
  const int k1 = kk + 8 * (g / 2) + i / 4, k2 = k1 + 4;
  const int c = n / 8, e = n % 8;
  const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)(s + k1 * R + ((c ^ kswz<R>(k1)) << 3) + e));
  const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)(s + k2 * R + ((c ^ kswz<R>(k2)) << 3) + e));
  u32x4 v;
  v[0] = (uint32_t)(uint16_t)r1[0] | ((uint32_t)(uint16_t)r1[1] << 16);
  v[1] = (uint32_t)(uint16_t)r1[2] | ((uint32_t)(uint16_t)r1[3] << 16);
  v[2] = (uint32_t)(uint16_t)r2[0] | ((uint32_t)(uint16_t)r2[1] << 16);
  v[3] = (uint32_t)(uint16_t)r2[2] | ((uint32_t)(uint16_t)r2[3] << 16);
  return v;
}

// One 64-deep K slice from LDS into the wave's accumulators.  AKM / BKM:
// operand staged k-major (else row-major, read transposed).  The layouts are
// template parameters so the slice is straight-line code: every fragment read
// of the slice is issued before the first MFMA, and the reads of later k steps
// overlap the MFMAs of earlier ones (with one wave per SIMD nothing else hides
// the LDS latency).
template <int BM, int BN, bool BF16, bool AKM, bool BKM>
DEV void mfma_slice(uint32_t tid, const LDS uint16_t* sa, const LDS uint16_t* sb, f32x16 (&acc)[BM / 64][BN / 64]) {
  constexpr int FM = BM / 64, FN = BN / 64, KS = kBK / 16;
  const int wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  u32x4 af[KS][FM], bfr[KS][FN];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int i = 0; i < FM; ++i) af[ks][i] = frag<BM, AKM>(tid, sa, wm * (BM / 2) + i * 32, ks * 16);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[ks][j] = frag<BN, BKM>(tid, sb, wn * (BN / 2) + j * 32, ks * 16);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<BF16>(af[ks][i], bfr[ks][j], acc[i][j]);
}

// The fragments of k step `ks` (16 deep) of a staged slice, for this wave's
// (BM/2) x (BN/2) block.
template <int BM, int BN, bool AKM, bool BKM>
DEV void read_frags(uint32_t tid, const LDS uint16_t* sa, const LDS uint16_t* sb, int ks, u32x4 (&fa)[BM / 64],
                    u32x4 (&fb)[BN / 64]) {
  const int wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
#pragma unroll
  for (int i = 0; i < BM / 64; ++i) fa[i] = frag<BM, AKM>(tid, sa, wm * (BM / 2) + i * 32, ks * 16);
#pragma unroll
  for (int j = 0; j < BN / 64; ++j) fb[j] = frag<BN, BKM>(tid, sb, wn * (BN / 2) + j * 32, ks * 16);
}

// Fast-path main loop (see gemm_mfma): a ring of S stages, S - 1 slices in
// flight, software-pipelined by 16-deep k steps: the fragments of step s + 1
// are read from LDS while the MFMAs of step s run (the two are interleaved
// in the instruction stream, so the LDS reads hide behind the matrix cores
// instead of preceding them).  At the last step of slice k the wave waits
// for slice k + 1, the workgroup meets (every wave has its fragments of slice
// k in registers and every wave's copy of slice k + 1 has landed), slice
// k + S is issued into slice k's stage, and the first fragments of slice
// k + 1 are read under the last MFMAs of slice k.  CS: also sum each of the
// wave's B fragments into bsum (lane l: column l % 32 of fragment j, the
// half of every k step that the lane holds).
template <int BM, int BN, bool BF16, bool AKM, bool BKM, int S, bool CS>
DEV void direct_loop(uint32_t tid, const DirectOp<BM>& da, const DirectOp<BN>& db, uint32_t nk,
                     f32x16 (&acc)[BM / 64][BN / 64], float (&bsum)[BN / 64]) {
  constexpr int FM = BM / 64, FN = BN / 64, KS = kBK / 16;
  constexpr int SA = BM * kBK * 2, SB = BN * kBK * 2;
  constexpr int LPS = BM / 32 + BN / 32;  // direct loads per wave per slice
  constexpr int NMF = FM * FN;            // MFMAs per k step
  constexpr int NDS = FM * (AKM ? 1 : 2) + FN * (BKM ? 1 : 2);  // LDS reads per k step
  constexpr int DPM = (NDS + NMF - 1) / NMF;                    // LDS reads between two MFMAs
  const uint32_t last = nk - 1;
  // slices 0 .. S-2 in flight (past the last slice, loads repeat it into a
  // stage that is not read again)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    const uint32_t sl = (uint32_t)s < last ? (uint32_t)s : last;
    da.issue(sl, s * (SA + SB));
    db.issue(sl, s * (SA + SB) + SA);
  }
  wait_vmcnt<(S - 2) * LPS>();  // this wave's copy of slice 0 has landed
  __syncthreads();              // ... and every wave's
  {
    const uint32_t sl = (uint32_t)(S - 1) < last ? (uint32_t)(S - 1) : last;
    da.issue(sl, (S - 1) * (SA + SB));
    db.issue(sl, (S - 1) * (SA + SB) + SA);
  }
  u32x4 fa[2][FM], fb[2][FN];
  read_frags<BM, BN, AKM, BKM>(tid, (const LDS uint16_t*)g_smem, (const LDS uint16_t*)(g_smem + SA), 0, fa[0], fb[0]);
  for (uint32_t k = 0; k < nk; ++k) {
    const uint32_t cs = (k % S) * (SA + SB);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
        read_frags<BM, BN, AKM, BKM>(tid, (const LDS uint16_t*)(g_smem + cs), (const LDS uint16_t*)(g_smem + cs + SA),
                                     ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
      } else {
        // slice k + 1: this wave's copy has landed once at most the S-2
        // younger slices are in flight; the barrier (which first waits for
        // this wave's fragment reads) covers every wave's copy and every
        // wave's last read of slice k, whose stage the next issue refills.
        // After the last slice this runs too, without branching (the loads
        // repeat the last slice into a stage that is not read again, and the
        // fragments read are not used), so the step stays one basic block in
        // which the reads interleave with the MFMAs.
        wait_vmcnt<(S - 2) * LPS>();
        __syncthreads();
        const uint32_t nx = k + S < last ? k + S : last;
        da.issue(nx, cs);
        db.issue(nx, cs + SA);
        const uint32_t ns = ((k + 1) % S) * (SA + SB);
        read_frags<BM, BN, AKM, BKM>(tid, (const LDS uint16_t*)(g_smem + ns), (const LDS uint16_t*)(g_smem + ns + SA),
                                     0, fa[cur ^ 1], fb[cur ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<BF16>(fa[cur][i], fb[cur][j], acc[i][j]);
      if constexpr (CS) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bsum[j] = frag_sum<BF16>(fb[cur][j], bsum[j]);
      }
      // interleave: MFMA, DPM fragment reads, MFMA, ...
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, DPM, 0);
      }
    }
  }
  wait_vmcnt<0>();  // no load may still be writing the arena
  __syncthreads();  // every wave is done with the ring (the C tile reuses it)
}

// Fast-path main loop of a 64x64 tile.  Each wave owns a 32x32 block, one
// MFMA per 16-deep k step, so a single accumulator would chain every MFMA
// on the previous one's result; instead k step s of every slice accumulates
// into partial sum s % 4 (four independent chains), and the partials are
// added in a fixed order at the end.  The fragments are double-buffered by
// slice: all of slice k + 1's fragments are read from LDS while slice k's
// four MFMAs run.  CS: as in direct_loop.
template <bool BF16, bool AKM, bool BKM, int S, bool CS>
DEV void direct_loop64(uint32_t tid, const DirectOp<64>& da, const DirectOp<64>& db, uint32_t nk,
                       f32x16 (&acc)[1][1], float (&cs)[1]) {
  constexpr int KS = kBK / 16;
  constexpr int SA = 64 * kBK * 2, SB = 64 * kBK * 2;
  constexpr int LPS = 4;                                  // direct loads per wave per slice
  constexpr int NDS = KS * ((AKM ? 1 : 2) + (BKM ? 1 : 2));  // LDS reads per slice
  constexpr int DPM = NDS / KS;                            // LDS reads between two MFMAs
  const int wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  const uint32_t last = nk - 1;
  f32x16 part[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) part[q][r] = 0.0f;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    const uint32_t sl = (uint32_t)s < last ? (uint32_t)s : last;
    da.issue(sl, s * (SA + SB));
    db.issue(sl, s * (SA + SB) + SA);
  }
  wait_vmcnt<(S - 2) * LPS>();
  __syncthreads();
  {
    const uint32_t sl = (uint32_t)(S - 1) < last ? (uint32_t)(S - 1) : last;
    da.issue(sl, (S - 1) * (SA + SB));
    db.issue(sl, (S - 1) * (SA + SB) + SA);
  }
  u32x4 fa[2][KS], fb[2][KS];
  auto read_slice = [&](uint32_t stage, u32x4 (&a)[KS], u32x4 (&b)[KS]) {
    const LDS uint16_t* sa = (const LDS uint16_t*)(g_smem + stage * (SA + SB));
    const LDS uint16_t* sb = (const LDS uint16_t*)(g_smem + stage * (SA + SB) + SA);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a[ks] = frag<64, AKM>(tid, sa, wm * 32, ks * 16);
      b[ks] = frag<64, BKM>(tid, sb, wn * 32, ks * 16);
    }
  };
  read_slice(0, fa[0], fb[0]);
  // slice k: with slice k + 1 landed and every wave's fragments of slice k in
  // registers, refill slice k's stage with slice k + S, read slice k + 1's
  // fragments, and run slice k's MFMAs under those reads
  // (after the last slice this runs too, without branching: the loads repeat
  // the last slice into a stage that is not read again and the fragments
  // read are not used, so the body stays one basic block in which the reads
  // interleave with the MFMAs)
  auto body = [&](uint32_t k, auto cur) {
    constexpr int C = decltype(cur)::value;
    {
      wait_vmcnt<(S - 2) * LPS>();
      __syncthreads();
      const uint32_t nx = k + S < last ? k + S : last;
      const uint32_t cs = (k % S) * (SA + SB);
      da.issue(nx, cs);
      db.issue(nx, cs + SA);
      read_slice((k + 1) % S, fa[C ^ 1], fb[C ^ 1]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) part[ks] = mfma32<BF16>(fa[C][ks], fb[C][ks], part[ks]);
    if constexpr (CS) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) cs[0] = frag_sum<BF16>(fb[C][ks], cs[0]);
    }
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, DPM, 0);
    }
  };
  uint32_t k = 0;
  for (; k + 1 < nk; k += 2) {
    body(k, std::integral_constant<int, 0>());
    body(k + 1, std::integral_constant<int, 1>());
  }
  if (k < nk) body(k, std::integral_constant<int, 0>());
  wait_vmcnt<0>();  // no load may still be writing the arena
  __syncthreads();  // every wave is done with the ring (the C tile reuses it)
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][0][r] = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
}

// BF16: operand dtype (bf16, else f16), a template parameter so the MFMA
// accumulators never change registers between the two instruction forms.
// before_loop() runs once the tile's coordinates are in `st`, before the
// first operand load: its loads complete ahead of the ring's (loads retire in
// issue order) and land in the arena above the ring.  Returns whether B's
// column sums came out of the main loop (then they are in the C tile's
// padding, see the end).
template <int BM, int BN, bool BF16, class BeforeLoop>
DEV bool gemm_mfma(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t item, ItemState& st,
                   BeforeLoop before_loop) {
  constexpr int FM = BM / 64, FN = BN / 64;  // 32x32 blocks per wave along m / n
  constexpr int S = BM == 128 ? 3 : 4;       // ring stages (S * (BM + BN) * 128 bytes <= the arena)
  constexpr int SA = BM * kBK * 2, SB = BN * kBK * 2;
  static_assert(S * (SA + SB) <= (int)(BM == 128 ? kFastStage128 : kFastStage64),
                "the operand ring overlaps the register epilogue's staged operands");
  static_assert(BM * (BN + 4) * 4 <= S * (SA + SB), "the C tile exceeds the operand ring");
  const uint32_t tiles = t.tiles_m * t.tiles_n;
  const uint32_t split_index = item / tiles;
  const uint32_t tile = xcd_tile(item % tiles, tiles);
  uint32_t tm, tn;
  tile_coords(t, tile, tm, tn);
  const uint32_t m0 = tm * BM, n0 = tn * BN;
  st.m0 = m0;
  st.n0 = n0;
  st.bm = BM;
  st.bn = BN;
  st.split_index = split_index;
  before_loop();
  const uint32_t kbeg = split_index * t.kchunk;
  const uint32_t kend = (kbeg + t.kchunk < t.k) ? kbeg + t.kchunk : t.k;
  const VView A = load_view(views_off + t.va * sizeof(DView)), B = load_view(views_off + t.vb * sizeof(DView));
  const GLOBAL uint16_t* pa = (const GLOBAL uint16_t*)base_ptr(ka, A.base);
  const GLOBAL uint16_t* pb = (const GLOBAL uint16_t*)base_ptr(ka, B.base);
  const int wave = tid / 64, lane = tid % 64;
  const int wm = wave / 2, wn = wave % 2;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const uint32_t nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
  // A's element (m, k) at off + m * stride[0] + k * stride[1];
  // B's element (n, k) at off + k * stride[0] + n * stride[1]
  const bool full_k = (kend - kbeg) % kBK == 0;
  const bool a_kc = A.stride[1] == 1, a_rc = !a_kc && A.stride[0] == 1;
  const bool b_kc = B.stride[0] == 1, b_rc = !b_kc && B.stride[1] == 1;
  const int64_t a_other = a_kc ? A.stride[0] : A.stride[1], b_other = b_kc ? B.stride[1] : B.stride[0];
  const bool a_ok = m0 + BM <= t.m && (a_kc || a_rc) && aligned16(pa) && (A.offset & 7) == 0 && (a_other & 7) == 0;
  const bool b_ok = n0 + BN <= t.n && (b_kc || b_rc) && aligned16(pb) && (B.offset & 7) == 0 && (b_other & 7) == 0;
  // B's column sums over all of K come out of the main loop for the first
  // tile row of a product that carries them (A and B staged row-major, the
  // whole of K in one part)
  float cs[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) cs[j] = 0.0f;
  const bool direct = nk > 0 && full_k && a_ok && b_ok;
  const bool csum = direct && (t.flags & F_BSUM) && (t.flags & F_FASTEPI) && m0 == 0 && !a_kc && !b_kc &&
                    kbeg == 0 && kend == t.k;
  if (direct) {
    DirectOp<BM> da;
    DirectOp<BN> db;
    da.init(tid, a_kc, pa, A.offset, A.stride[0], A.stride[1], m0, kbeg);
    db.init(tid, b_kc, pb, B.offset, B.stride[1], B.stride[0], n0, kbeg);
    if constexpr (BM == 64 && BN == 64) {
      if (a_kc) {
        if (b_kc)
          direct_loop64<BF16, true, true, S, false>(tid, da, db, nk, acc, cs);
        else
          direct_loop64<BF16, true, false, S, false>(tid, da, db, nk, acc, cs);
      } else {
        if (b_kc)
          direct_loop64<BF16, false, true, S, false>(tid, da, db, nk, acc, cs);
        else if (csum)
          direct_loop64<BF16, false, false, S, true>(tid, da, db, nk, acc, cs);
        else
          direct_loop64<BF16, false, false, S, false>(tid, da, db, nk, acc, cs);
      }
    } else if (a_kc) {
      if (b_kc)
        direct_loop<BM, BN, BF16, true, true, S, false>(tid, da, db, nk, acc, cs);
      else
        direct_loop<BM, BN, BF16, true, false, S, false>(tid, da, db, nk, acc, cs);
    } else {
      if (b_kc)
        direct_loop<BM, BN, BF16, false, true, S, false>(tid, da, db, nk, acc, cs);
      else if (csum)
        direct_loop<BM, BN, BF16, false, false, S, true>(tid, da, db, nk, acc, cs);
      else
        direct_loop<BM, BN, BF16, false, false, S, false>(tid, da, db, nk, acc, cs);
    }
  } else {
    LDS uint16_t* sa0 = (LDS uint16_t*)g_smem;
    LDS uint16_t* sb0 = (LDS uint16_t*)(g_smem + SA);
    for (uint32_t kt = 0; kt < nk; ++kt) {
      const uint32_t k0 = kbeg + kt * kBK;
      slow_stage<BM>(tid, pa, A.offset, A.stride[0], A.stride[1], m0, t.m, k0, kend, sa0);
      slow_stage<BN>(tid, pb, B.offset, B.stride[1], B.stride[0], n0, t.n, k0, kend, sb0);
      __syncthreads();
      mfma_slice<BM, BN, BF16, true, true>(tid, sa0, sb0, acc);
      __syncthreads();
    }
  }
  // accumulators -> LDS tile [BM][BN + 4]
  LDS float* C = (LDS float*)g_smem;
  const int pitch = BN + 4;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / 2) + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
        const int col = wn * (BN / 2) + j * 32 + (lane % 32);
        C[row * pitch + col] = acc[i][j][r];
      }
  // column sums -> the tile's padding: column c's two halves at padding
  // slots 2c and 2c + 1 (slot p at row p / 4, column BN + p % 4)
  if (csum && uniform((uint32_t)wm) == 0) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int p = 2 * (wn * (BN / 2) + j * 32 + lane % 32) + lane / 32;
      C[(p / 4) * pitch + BN + p % 4] = cs[j];
    }
  }
  return csum;
}

// ------------------------------------------------------ int8-weight GEMV --
// 16 output rows per work item, 4 per wave; each lane takes 16-wide K chunks
// (k = 16 * lane + 1024 * j).  All weight loads of a wave's 4 rows for up to
// 4096 columns are issued before any is used.  w = fl(q * s), then
// acc = fma(x, w, acc).  Leaves the 16 row sums in LDS.

// One DPP step: v + (v moved across lanes by `ctrl`) in the rows of
// `rows` (other rows add zero).
template <int ctrl, int rows>
DEV float dpp_add(float v) {
  const int m = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rows, 0xf, false);
  return v + __builtin_bit_cast(float, m);
}

// Sum over the 64 lanes of a wave, in a fixed order, on DPP lane moves
// instead of LDS permutes: lane pairs, quads, 16-lane rows (two rotations),
// then the rows combined by broadcasts (row 0 into row 1 and row 2 into row 3,
// then rows 0+1 into row 3).  The total is read from lane 63 (wave-uniform).
DEV float wave_sum(float v) {
  v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x124, 0xf>(v);  // row_ror:4
  v = dpp_add<0x128, 0xf>(v);  // row_ror:8
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

constexpr uint32_t kGemvRed = kSmemBytes - 64 * kGemvRows;  // byte offset of the [rows][16] output sums

// Split-K GEMV slab: output columns cb*16 .. +16 (rows of the int8 weight q,
// four per wave) for activation rows r0 .. r0+R-1.  Each lane takes 16-wide
// K chunks; the weight chunks are loaded once and serve all R rows.
template <int R>
DEV void gemv_q8_rows(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t cb, uint32_t r0) {
  const VView X = load_view(views_off + t.va * sizeof(DView)), Q = load_view(views_off + t.vb * sizeof(DView)),
              S = load_view(views_off + t.vs * sizeof(DView));
  const GLOBAL uint8_t* px = base_ptr(ka, X.base);
  const GLOBAL int8_t* pq = (const GLOBAL int8_t*)base_ptr(ka, Q.base);
  const GLOBAL float* ps = (const GLOBAL float*)base_ptr(ka, S.base);
  const int wave = tid / 64, lane = tid % 64;
  const uint32_t K = t.k;
  LDS float* xs = (LDS float*)g_smem;  // [R][K] activations, when staged
  // A contiguous, 16-byte aligned bf16 row is read straight into registers
  // (each lane needs only its own 64 values): no staging, and none of the
  // bank conflicts of lane-strided LDS reads.
  const GLOBAL uint16_t* xrow = (const GLOBAL uint16_t*)px + X.offset + (int64_t)r0 * X.stride[0];
  const bool xreg = R == 1 && X.dtype == DT_BF16 && X.stride[1] == 1 && K % 16 == 0 && aligned16(xrow);
  const bool staged = !xreg && (uint64_t)K * 4 * R <= (uint64_t)kGemvRed;
  const uint32_t row0 = cb * 16 + wave * 4;
  // Fast form (uniform per task): contiguous int8 rows, 16-byte aligned
  // chunk starts, K a multiple of 16.  Every load is then issued
  // unconditionally from a clamped in-bounds address, so all sixteen chunks
  // of a lane are in flight at once; lanes past the end mask the weights
  // when they use them.
  const bool fast = (staged || xreg) && Q.stride[1] == 1 && K % 16 == 0 && (Q.offset & 15) == 0 &&
                    (Q.stride[0] & 15) == 0 && aligned16(pq);
  constexpr int NC = 4;  // chunks per lane per pass (4096 columns)
  float acc[4][R];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.0f;
  for (uint32_t kpass = 0; kpass < K; kpass += 1024 * NC) {
    u32x4 qv[4][NC];
    float sv[4][NC];
    uint32_t okm = 0;  // bit i * NC + j: chunk (i, j) exists
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = row0 + i;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const uint32_t kc = kpass + 1024 * j + lane * 16;
        okm |= (row < t.n && kc < K ? 1u : 0u) << (i * NC + j);
      }
    }
    if (fast) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = row0 + i < t.n ? row0 + i : 0;
        const int64_t qrow = Q.offset + (int64_t)row * Q.stride[0];
        const int64_t srow = S.offset + (int64_t)row * S.stride[0];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const uint32_t kc0 = kpass + 1024 * j + lane * 16;
          const uint32_t kc = kc0 < K ? kc0 : 0;
          qv[i][j] = *(const GLOBAL u32x4*)(pq + qrow + kc);
          // a 16-wide chunk starting at a multiple of 16 lies inside one 32-block
          sv[i][j] = ps[srow + (int64_t)(kc / 32) * S.stride[1]];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = row0 + i;
        const int64_t qrow = Q.offset + (int64_t)row * Q.stride[0];
        const int64_t srow = S.offset + (int64_t)row * S.stride[0];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const uint32_t kc = kpass + 1024 * j + lane * 16;
          const bool ok = (okm >> (i * NC + j)) & 1u;
          const int64_t qidx = qrow + (int64_t)kc * Q.stride[1];
          uint32_t w[4] = {0, 0, 0, 0};
          for (int e = 0; e < 16; ++e)
            if (ok && kc + e < K) w[e / 4] |= ((uint32_t)(uint8_t)pq[qidx + (int64_t)e * Q.stride[1]]) << (8 * (e % 4));
          qv[i][j] = u32x4{w[0], w[1], w[2], w[3]};
          sv[i][j] = ok ? ps[srow + (int64_t)(kc / 32) * S.stride[1]] : 0.0f;
        }
      }
    }
    u32x4 xr[NC][2];  // xreg: this lane's 16 bf16 activations per chunk
    if (xreg) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const uint32_t kc0 = kpass + 1024 * j + lane * 16;
        const GLOBAL u32x4* xp = (const GLOBAL u32x4*)(xrow + (kc0 < K ? kc0 : 0));
        xr[j][0] = xp[0];
        xr[j][1] = xp[1];
      }
    }
    if (kpass == 0 && staged) {
      // 16 elements per thread and row per round, every load issued before
      // any is stored (one latency per round, not one per element)
      for (int r = 0; r < R; ++r)
        for (uint32_t k0 = 0; k0 < K; k0 += 16 * kBlock) {
          const int64_t rb = X.offset + (int64_t)(r0 + r) * X.stride[0];
          float v[16];
          if (X.dtype == DT_F32) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const uint32_t k = k0 + tid + kBlock * u;
              v[u] = ((const GLOBAL float*)px)[rb + (int64_t)(k < K ? k : 0) * X.stride[1]];
            }
          } else if (X.dtype == DT_I8) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const uint32_t k = k0 + tid + kBlock * u;
              v[u] = (float)((const GLOBAL int8_t*)px)[rb + (int64_t)(k < K ? k : 0) * X.stride[1]];
            }
          } else {
            uint32_t h[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const uint32_t k = k0 + tid + kBlock * u;
              h[u] = ((const GLOBAL uint16_t*)px)[rb + (int64_t)(k < K ? k : 0) * X.stride[1]];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = half_bits_to_f32(h[u], X.dtype == DT_BF16);
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const uint32_t k = k0 + tid + kBlock * u;
            if (k < K) xs[r * K + k] = v[u];
          }
        }
      __syncthreads();
    }
    if (t.flags & F_XQ) {
      // Q8_0 activations: the two lanes of a 32-block exchange their
      // absolute maxima, d = amax / 127, codes round(x / d) (ties to even;
      // d = 0 gives codes 0), then per weight row an exact integer dot of
      // the lane's 16 codes with its 16 weight bytes, weighted by d * s.
      // The quotients are correctly rounded divisions, as on the CPU side.
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const uint32_t kc = kpass + 1024 * j + lane * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float xk[16], amax = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t xi = X.offset + (int64_t)(r0 + r) * X.stride[0] + (int64_t)(kc + e) * X.stride[1];
            if (xreg) {
              const uint32_t w = xr[j][e / 8][(e % 8) / 2];
              xk[e] = kc < K ? __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)) : 0.0f;
            } else {
              xk[e] = (kc + e < K) ? (staged ? xs[r * K + kc + e] : load_elem(px, X.dtype, xi)) : 0.0f;
            }
            amax = fmaxf(amax, fabsf(xk[e]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
          const float d = amax / 127.0f;
          int32_t cw[4] = {0, 0, 0, 0};
          if (d != 0.0f) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float c = fminf(127.0f, fmaxf(-127.0f, __builtin_rintf(xk[e] / d)));
              cw[e / 4] |= ((int32_t)c & 0xff) << (8 * (e % 4));
            }
          }
          if (kc < K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              int32_t idot = 0;
#pragma unroll
              for (int w4 = 0; w4 < 4; ++w4) idot = __builtin_amdgcn_sdot4((int32_t)qv[i][j][w4], cw[w4], idot, false);
              const float wsc = d * sv[i][j];
              acc[i][r] = __builtin_fmaf(wsc, (float)idot, acc[i][r]);
            }
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const uint32_t kc = kpass + 1024 * j + lane * 16;
      if (kc >= K) continue;
      // q = b - 128 with b = q ^ 0x80 an unsigned byte (converted by the
      // byte-select conversions), so a chunk's dot product is
      // sum(x b) - 128 sum(x), scaled once by the block scale
      float xk[R][16], xoff[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float xsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t xi = X.offset + (int64_t)(r0 + r) * X.stride[0] + (int64_t)(kc + e) * X.stride[1];
          if (xreg) {
            const uint32_t w = xr[j][e / 8][(e % 8) / 2];
            xk[r][e] = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
          } else {
            xk[r][e] = (kc + e < K) ? (staged ? xs[r * K + kc + e] : load_elem(px, X.dtype, xi)) : 0.0f;
          }
          xsum = xsum + xk[r][e];
        }
        xoff[r] = 128.0f * xsum;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float wb[16];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t u = qv[i][j][w4] ^ 0x80808080u;
#pragma unroll
          for (int by = 0; by < 4; ++by) wb[4 * w4 + by] = (float)((u >> (8 * by)) & 0xffu);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float d = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) d = __builtin_fmaf(xk[r][e], wb[e], d);
          acc[i][r] = __builtin_fmaf(sv[i][j], d - xoff[r], acc[i][r]);
        }
      }
    }
  }
  LDS float* red = (LDS float*)(g_smem + kGemvRed);  // [R][16]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = wave_sum(acc[i][r]);
      if (lane == 0) red[r * 16 + wave * 4 + i] = s;
    }
  __syncthreads();
}

// Work item = slab * tiles_n + column block; a slab is kGemvRows activation
// rows (the last may be shorter).
DEV void gemv_q8(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t item) {
  const uint32_t cb = item % t.tiles_n, r0 = (item / t.tiles_n) * kGemvRows;
  const uint32_t rows = t.m - r0 < kGemvRows ? t.m - r0 : kGemvRows;
  switch (rows) {
    case 1: gemv_q8_rows<1>(tid, ka, t, views_off, cb, r0); break;
    case 2: gemv_q8_rows<2>(tid, ka, t, views_off, cb, r0); break;
    case 3: gemv_q8_rows<3>(tid, ka, t, views_off, cb, r0); break;
    default: gemv_q8_rows<4>(tid, ka, t, views_off, cb, r0); break;
  }
}

// Block-wide sum in a fixed order: wave butterflies, then waves 0..3 in order.
DEV float block_sum(uint32_t tid, float v) {
  LDS float* scratch = (LDS float*)g_smem;
  v = wave_sum(v);
  const int wave = tid / 64, lane = tid % 64;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float s = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
  __syncthreads();
  return s;
}

// -------------------------------------------------------------- batches --

DEV void set_1d(Batch& b, uint32_t d0) {
  b.dims[0] = d0;
#pragma unroll
  for (int d = 1; d < kMaxDims; ++d) {
    b.dims[d] = 1;
    b.dmul[d] = 1;
    b.dsh[d] = 0;
  }
  b.nd = 1;
}

DEV void expr_batch(Batch& b, const DTask& t, uint32_t ins_off) {
  b.ins = ins_off + t.expr_first * sizeof(DIns);
  b.n = t.expr_len;
  b.width = t.width == 8 ? 8 : 1;
  b.accumulate = 0;
}

DEV void task_space(Batch& b, const DTask& t) {
  b.nd = t.ndim;
#pragma unroll
  for (int d = 0; d < kMaxDims; ++d) {
    b.dims[d] = t.dims[d];
    b.dmul[d] = t.dmul[d];
    b.dsh[d] = t.dsh[d];
  }
}

DEV void fin_batch(Batch& b, const DTask& t, uint32_t ins_off, uint32_t width) {
  b.ins = ins_off + t.fin_first * sizeof(DIns);
  b.n = t.fin_len;
  b.width = width;
  b.accumulate = 0;
  set_1d(b, t.m);
}

// ------------------------------------------------- one-element programs --
// A program evaluated for one element per thread, in registers, with
// vm_run's arithmetic and rounding instruction by instruction (so results are
// identical bit for bit): for work with too few elements per thread for the
// batches' chunk machinery to pay (the int8 GEMV's epilogue, the finishing
// programs of reductions).  `ins` is the byte offset of the first instruction
// in the LDS plan; c holds the element's coordinates (views index with
// them); stores are skipped where ok is false.  Slots are this thread's word
// of the LDS slot arrays.
//
// The operand loads that come before the program's first store may be issued
// ahead of the work that produces y (prog_preload, up to kPre of them): no
// store of the program precedes them and the callers' work writes no memory
// until the program runs.  Operand k lands in raw[k] as loaded (fp32 bits,
// the 16-bit pattern of an f16/bf16, or the sign-extended int8): nothing
// reads it before prog_run, so no wait for it is placed ahead of that work.
constexpr int kPre = 4;

DEV uint32_t prog_preload(const Ctx& ka, uint32_t views_off, uint32_t ins, uint32_t n_ins,
                          const uint32_t (&c)[kMaxDims], uint32_t (&raw)[kPre]) {
  uint32_t n = 0, pc = 0;
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    // the next operand load before the first store, if any (wave-uniform)
    uint32_t arg = 0xffffffffu;
    for (; pc < n_ins; ++pc) {
      const LDS uint32_t* iw = (const LDS uint32_t*)(g_plan + ins + pc * sizeof(DIns));
      const uint32_t w0 = uniform(iw[0]);
      if ((w0 & 0xff) == VM_STORE) {
        pc = n_ins;
        break;
      }
      if (((w0 >> 8) & 0xff) == SRC_VIEW) {
        arg = uniform(iw[1]) & 0xffff;
        ++pc;
        break;
      }
    }
    if (arg == 0xffffffffu) break;
    const VView v = load_view(views_off + arg * sizeof(DView));
    const GLOBAL uint8_t* p = base_ptr(ka, v.base);
    const int32_t idx = view_index(v, c);
    if (v.dtype == DT_F32)
      raw[k] = ((const GLOBAL uint32_t*)p)[idx];
    else if (v.dtype == DT_I8)
      raw[k] = (uint32_t)(int32_t)((const GLOBAL int8_t*)p)[idx];
    else
      raw[k] = ((const GLOBAL uint16_t*)p)[idx];
    ++n;
  }
  return n;
}

DEV void prog_run(uint32_t tid, const Ctx& ka, uint32_t views_off, uint32_t ins, uint32_t n_ins,
                  const uint32_t (&c)[kMaxDims], bool ok, float y, const uint32_t (&raw)[kPre], uint32_t npre) {
  uint32_t used = 0;  // preloaded operands consumed (in program order)
  for (uint32_t pc = 0; pc < n_ins; ++pc) {
    const LDS uint32_t* iw = (const LDS uint32_t*)(g_plan + ins + pc * sizeof(DIns));
    const uint32_t w0 = uniform(iw[0]), w1 = uniform(iw[1]);
    const float a = __uint_as_float(uniform(iw[2])), sv = __uint_as_float(uniform(iw[3]));
    const uint32_t op = w0 & 0xff, src = (w0 >> 8) & 0xff, rnd = (w0 >> 16) & 0xff, rev = w0 >> 24;
    const uint32_t arg = w1 & 0xffff;
    float o = 0.0f;
    if (src == SRC_VIEW || op == VM_STORE) {
      const VView v = load_view(views_off + arg * sizeof(DView));
      GLOBAL uint8_t* p = base_ptr(ka, v.base);
      const int32_t idx = view_index(v, c);
      if (op == VM_STORE) {
        if (ok) {
          if (v.dtype == DT_F32)
            ((GLOBAL float*)p)[idx] = y;
          else if (v.dtype != DT_I8)
            ((GLOBAL uint16_t*)p)[idx] = (uint16_t)f32_to_half_bits(y, v.dtype == DT_BF16);
        }
        continue;
      }
      if (used < npre) {
        uint32_t bits = raw[0];
#pragma unroll
        for (int k = 1; k < kPre; ++k)
          if ((uint32_t)k == used) bits = raw[k];
        o = v.dtype == DT_F32 ? __uint_as_float(bits)
            : v.dtype == DT_I8 ? (float)(int32_t)bits
                               : half_bits_to_f32(bits, v.dtype == DT_BF16);
        ++used;
      } else {
        o = load_elem(p, v.dtype, idx);
      }
    } else if (src == SRC_SLOT) {
      o = slot_base(arg)[tid];
    } else if (src == SRC_SCALAR) {
      o = sv;
    }
    switch (op) {
      case VM_LOAD: y = o; break;
      case VM_ADD:
        if (rev) { const float u = a * y; y = o + u; }
        else { const float u = a * o; y = y + u; }
        break;
      case VM_SUB:
        if (rev) { const float u = a * y; y = o - u; }
        else { const float u = a * o; y = y - u; }
        break;
      case VM_MUL: y = y * o; break;
      case VM_DIV: y = rev ? o / y : y / o; break;
      case VM_NEG: y = -y; break;
      case VM_RELU: y = y < 0.0f ? 0.0f : y; break;
      case VM_SQUARE: y = y * y; break;
      case VM_POW: y = powf(y, a); break;
      case VM_TB:
        if (rev) y = y <= a ? 0.0f : o;
        else y = o <= a ? 0.0f : y;
        break;
      case VM_SAVE: slot_base(arg)[tid] = y; break;
      case VM_SCALE: y = a * y; break;
      case VM_ZERO: y = 0.0f; break;
      case VM_SQRT: y = sqrtf(y); break;
      default: break;
    }
    if (rnd == DT_BF16)
      y = bf16_bits_to_f32(f32_to_bf16_bits(y));
    else if (rnd == DT_F16)
      y = f16_bits_to_f32(f32_to_f16_bits(y));
  }
}

// Coordinates of the int8 GEMV item's output for this thread of wave 0:
// output (r0 + tid / 16, cb * 16 + tid % 16); threads without one address
// element 0.
DEV bool gemv_out_coords(uint32_t tid, const DTask& t, uint32_t ins_off, uint32_t item, uint32_t (&c)[kMaxDims]) {
  const uint32_t cb = item % t.tiles_n, r0 = (item / t.tiles_n) * kGemvRows;
  const uint32_t rows = t.m - r0 < kGemvRows ? t.m - r0 : kGemvRows;
  const uint32_t r = tid / 16, col = cb * 16 + tid % 16;
  const bool ok = r < rows && col < t.n;
  Batch b;
  expr_batch(b, t, ins_off);
  task_space(b, t);
  unravel(ok ? (r0 + r) * t.n + col : 0u, b, c);
  return ok;
}

// The GEMV epilogue's leading operand loads, issued by wave 0 before the
// product (the product writes no memory).
DEV uint32_t gemv_epi_preload(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t ins_off,
                              uint32_t item, uint32_t (&raw)[kPre]) {
  if (tid >= 64) return 0;
  uint32_t c[kMaxDims];
  gemv_out_coords(tid, t, ins_off, item, c);
  return prog_preload(ka, views_off, ins_off + t.expr_first * sizeof(DIns), t.expr_len, c, raw);
}

// Epilogue of an int8-weight GEMV item: its 16 x rows outputs, one per thread
// of wave 0, from the row sums in LDS.
DEV void gemv_epilogue(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t views_off, uint32_t ins_off,
                       uint32_t item, const uint32_t (&raw)[kPre], uint32_t npre) {
  if (tid >= 64) return;
  uint32_t c[kMaxDims];
  const bool ok = gemv_out_coords(tid, t, ins_off, item, c);
  const LDS float* red = (const LDS float*)(g_smem + kGemvRed);
  const float y = ok ? red[(tid / 16) * 16 + tid % 16] : 0.0f;
  prog_run(tid, ka, views_off, ins_off + t.expr_first * sizeof(DIns), t.expr_len, c, ok, y, raw, npre);
}

// A contraction tile's batch (chunks q0 + q * kBlock + tid of the [bm][bn]
// tile, W elements each) into the exchange, or its split-K partial into the
// workspace.  All tile reads are issued before the exchange writes.  Returns
// the live-chunk mask.
template <int W>
DEV uint32_t fill_tile(uint32_t tid, const Ctx& ka, const DTask& t, const ItemState& st, int q0) {
  constexpr int C = kVmElems / W;
  const int pitch = st.bn + 4;
  const int lcpr = __builtin_ctz((uint32_t)(st.bn / W));  // log2 chunks per row
  const int nchunks = st.bm << lcpr;
  const LDS float* ctile = (const LDS float*)g_smem;
  float v[C][W];
  uint32_t e[C];
  bool ok[C], in[C];
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const int qq = q0 + q * kBlock + (int)tid;
    in[q] = qq < nchunks;
    const int r = in[q] ? qq >> lcpr : 0, cc = in[q] ? (qq & ((1 << lcpr) - 1)) * W : 0;
    const uint32_t row = st.m0 + r, col = st.n0 + cc;
    ok[q] = in[q] && row < t.m && col < t.n;
    e[q] = ok[q] ? row * t.n + col : 0;
    const LDS float* src = ctile + r * pitch + cc;
    if constexpr (W == 8) {
      // rows are 16-byte aligned (pitch a multiple of 4) and chunks start at
      // multiples of 8 columns
      const u32x4 a = *(const LDS u32x4*)src, c = *(const LDS u32x4*)(src + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[q][j] = __uint_as_float(a[j]);
        v[q][4 + j] = __uint_as_float(c[j]);
      }
    } else {
      v[q][0] = *src;
    }
  }
  if (t.flags & F_PARTIAL) {
    GLOBAL float* P = ws_f32(ka, t.scratch) + (uint64_t)st.split_index * t.m * t.n;
#pragma unroll
    for (int q = 0; q < C; ++q)
      if (ok[q])
#pragma unroll
        for (int j = 0; j < W; ++j) P[e[q] + j] = v[q][j];
    return 0u;
  }
  uint32_t live = 0;
#pragma unroll
  for (int q = 0; q < C; ++q) {
    live |= (ok[q] ? 1u : 0u) << q;
    xe(tid, q) = e[q];
#pragma unroll
    for (int j = 0; j < W; ++j) xv(tid, q * W + j) = in[q] ? v[q][j] : 0.0f;
  }
  return live;
}

// Fill batch `bi` of a work item: set up the program and the exchange, and
// set this thread's live-chunk mask.  Returns false when the item has no
// batch `bi` (uniform across the workgroup).
DEV bool fill(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t ins_off, uint32_t item, uint32_t bi, ItemState& st, Batch& b,
              uint32_t& live) {
  live = 0;
  // every chunk index must address the iteration space: dead chunks read
  // element 0 (the machine loads every chunk, and stores only live ones)
#pragma unroll
  for (int q = 0; q < kVmElems; ++q) xe(tid, q) = 0;
  const int W = t.width == 8 ? 8 : 1, C = kVmElems / W;
  switch (t.kind) {
    case T_EW: {
      // 4096 consecutive elements per item: two 8-wide chunks or sixteen singles per thread
      if (bi > 0) return false;
      expr_batch(b, t, ins_off);
      task_space(b, t);
      const uint32_t numel = t.dims[0] * t.dims[1] * t.dims[2] * t.dims[3];  // unused dims are 1
      const uint32_t base = item * 4096u;
      for (int q = 0; q < C; ++q) {
        const uint32_t e = W == 8 ? base + q * 2048u + tid * 8u : base + q * 256u + tid;
        xe(tid, q) = e < numel ? e : 0;
        live |= (e < numel ? 1u : 0u) << q;
      }
      for (int j = 0; j < kVmElems; ++j) xv(tid, j) = 0.0f;
      return true;
    }
    case T_GEMM_MFMA:
    case T_GEMM_SIMT: {
      // epilogue over the fp32 tile in LDS ([bm][bn + 4]), 16 elements per
      // thread per batch; split-K partial tiles are written out instead
      const int cpr = st.bn / W;  // chunks per row (a power of two)
      const int q0 = (int)bi * kBlock * C;
      if (q0 >= st.bm * cpr) return false;
      expr_batch(b, t, ins_off);
      task_space(b, t);
      if (W == 8)
        live = fill_tile<8>(tid, ka, t, st, q0);
      else
        live = fill_tile<1>(tid, ka, t, st, q0);
      return true;
    }
    case T_GEMM_REDUCE: {
      // split-K combine: partial tiles summed in split order, then the epilogue
      if (bi > 0) return false;
      expr_batch(b, t, ins_off);
      task_space(b, t);
      const uint64_t total = (uint64_t)t.m * t.n;
      const GLOBAL float* P = ws_f32(ka, t.scratch);
      for (int q = 0; q < C; ++q) {
        const uint64_t e = (uint64_t)item * 4096u + (W == 8 ? q * 2048u + tid * 8u : q * 256u + tid);
        const bool ok = e < total;
        live |= (ok ? 1u : 0u) << q;
        xe(tid, q) = ok ? (uint32_t)e : 0;
        for (int j = 0; j < W; ++j) {
          float a = ok ? P[e + j] : 0.0f;
          for (uint32_t s = 1; s < t.split; ++s) a = a + (ok ? P[s * total + e + j] : 0.0f);
          xv(tid, q * W + j) = a;
        }
      }
      return true;
    }
    case T_RED_ROWS: {
      // item = row * parts + part; thread t takes chunks t, t + 256, ... of
      // its part; the batch after the last sums over the block and finishes
      const uint32_t row = item / t.split, part = item % t.split;
      const uint32_t R = t.k;
      const uint32_t kb = part * t.kchunk;
      const uint32_t ke = (kb + t.kchunk < R) ? kb + t.kchunk : R;
      const uint32_t per = kBlock * W * C;
      const uint32_t nb = ke > kb ? (ke - kb + per - 1) / per : 0;
      if (bi < nb) {
        expr_batch(b, t, ins_off);
        task_space(b, t);
        b.accumulate = 1;
        const uint32_t k0 = kb + bi * per + tid * W;
        for (int q = 0; q < C; ++q) {
          const uint32_t kk = k0 + q * kBlock * W;
          const bool ok = kk < ke;
          live |= (ok ? 1u : 0u) << q;
          xe(tid, q) = row * R + (ok ? kk : kb);
        }
        for (int j = 0; j < kVmElems; ++j) xv(tid, j) = 0.0f;
        return true;
      }
      if (bi > nb) return false;
      const float total = block_sum(tid, st.acc);
      fin_batch(b, t, ins_off, 1);
      if (tid == 0) {
        if (t.flags & F_PARTIAL) {
          ws_f32(ka, t.scratch)[(uint64_t)row * t.split + part] = total;
        } else {
          live = 1;
          xe(tid, 0) = row;
          xv(tid, 0) = total;
        }
      }
      return true;
    }
    case T_RED_COLS: {
      // item = colblock * parts + part; 32 column chunks x 8 row lanes; rows
      // taken lane-strided, then summed across lanes in order
      const uint32_t cb = item / t.split, part = item % t.split;
      const uint32_t cols = t.m, R = t.k;
      const uint32_t cc = tid % 32, rl = tid / 32;
      const uint32_t col = cb * 32 * W + cc * W;
      const uint32_t rb = part * t.kchunk;
      const uint32_t re = (rb + t.kchunk < R) ? rb + t.kchunk : R;
      const uint32_t per = 8 * C;
      // (F_COLDIRECT items never come here: red_cols_item runs them)
      const uint32_t nb = re > rb ? (re - rb + per - 1) / per : 0u;
      if (bi < nb) {
        expr_batch(b, t, ins_off);
        task_space(b, t);
        b.accumulate = 1;
        const uint32_t r0 = rb + bi * per + rl;
        for (int q = 0; q < C; ++q) {
          const uint32_t r = r0 + 8 * q;
          const bool ok = r < re && col < cols;
          live |= (ok ? 1u : 0u) << q;
          xe(tid, q) = (ok ? r : rb) * cols + (col < cols ? col : 0);
        }
        for (int j = 0; j < kVmElems; ++j) xv(tid, j) = 0.0f;
        return true;
      }
      if (bi > nb) return false;
      LDS float* red = (LDS float*)g_smem;  // [8][32 * W]
      for (int j = 0; j < W; ++j) red[rl * 32 * W + cc * W + j] = st.acc8[j];
      __syncthreads();
      fin_batch(b, t, ins_off, W);
      if (rl == 0 && col < cols) {
        float tot[8];
        for (int j = 0; j < W; ++j) {
          float a = red[cc * W + j];
          for (int q = 1; q < 8; ++q) a = a + red[q * 32 * W + cc * W + j];
          tot[j] = a;
        }
        if (t.flags & F_PARTIAL) {
          GLOBAL float* P = ws_f32(ka, t.scratch) + (uint64_t)part * cols + col;
          for (int j = 0; j < W; ++j) P[j] = tot[j];
        } else {
          // finishing program over `cols` outputs: one 8-wide chunk or one element
          live = 1;
          xe(tid, 0) = col;
          for (int j = 0; j < W; ++j) xv(tid, j) = tot[j];
        }
      }
      return true;
    }
    default:
      return false;
  }
}

// After a summing batch: a reduction adds the machine's results into the
// thread's running sums (chunk by chunk, elements in order).
DEV void consume(uint32_t tid, const DTask& t, const Batch& b, uint32_t live, ItemState& st) {
  if (!b.accumulate) return;
  const int W = t.width == 8 ? 8 : 1, C = kVmElems / W;
  if (t.kind == T_RED_ROWS) {
    for (int q = 0; q < C; ++q)
      if (live & (1u << q))
        for (int j = 0; j < W; ++j) st.acc = st.acc + xv(tid, q * W + j);
  } else {
    for (int q = 0; q < C; ++q)
      if (live & (1u << q))
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < W) st.acc8[j] = st.acc8[j] + xv(tid, q * W + j);
  }
}

// ------------------------------------------------------ register epilogue --
// A contraction tile whose epilogue the scheduler marked F_FASTEPI runs it
// here instead of through machine batches: a straight-line program of at most
// kFastIns instructions over 8-wide column chunks of the fp32 tile in LDS
// (loads and stores of 2-D views over (row, col) with column stride 1, or 0
// for loads).  Every thread owns G chunks (chunk g * kBlock + tid of the
// tile: the whole tile in one pass) and carries their values in registers
// through the program to the stores.
//   * Before the main loop's first operand load, every loaded view with
//     column stride 1 is copied global -> LDS, each lane its own chunks, into
//     the arena above the operand ring (fast_prefetch): the copies are in
//     flight under the main loop, and the program reads its operands from LDS.
//   * The program runs from host-encoded records, two 16-byte words per
//     instruction (the instruction with its staged offset, and its view
//     resolved to base, dtype, offset and strides), one instruction at a
//     time: only the current record occupies scalar registers (a decoded copy
//     of the whole program does not fit them and spills).
// The arithmetic, its order and every rounding are vm_run's, so results are
// identical bit for bit.  Hoisting every load before the first store is
// safe for the programs the scheduler marks: no load reads bytes an earlier
// store of the program may write.

// Output coordinates of this thread's G chunks.
template <int G>
struct FastChunks {
  int32_t row[G], col[G];  // output coordinates
  int r[G], cc[G];         // tile-local row and first column
  bool ok[G];              // inside the output
};

template <int G>
DEV void fast_chunks(uint32_t tid, const DTask& t, const ItemState& st, FastChunks<G>& c) {
  const int lcpr = __builtin_ctz((uint32_t)(st.bn / 8));  // log2 chunks per row
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int qq = g * kBlock + (int)tid;  // < bm * bn / 8 == G * kBlock
    c.r[g] = qq >> lcpr;
    c.cc[g] = (qq & ((1 << lcpr) - 1)) * 8;
    c.row[g] = (int32_t)st.m0 + c.r[g];
    c.col[g] = (int32_t)st.n0 + c.cc[g];
    c.ok[g] = (uint32_t)c.row[g] < t.m && (uint32_t)c.col[g] < t.n;
  }
}

// One instruction of a register epilogue, from its record (plan.h): the
// instruction and its view resolved (wave-uniform).
struct FRec {
  uint32_t w0;       // op | src << 8 | rnd << 16 | rev << 24
  float a, s;
  uint32_t staged;   // byte offset of the view's staged chunks in the arena, or 0
  uint32_t base, dt, s1;
  int32_t off, s0;
};

DEV u32x4 frec_word(uint32_t ins_off, uint32_t slot) {
  return *(const LDS u32x4*)(g_plan + ins_off + slot * sizeof(DIns));
}

DEV FRec frec_decode(const u32x4& A, const u32x4& B) {
  FRec r;
  r.w0 = uniform(A[0]);
  const uint32_t pad = uniform(A[1]) >> 16;
  r.staged = pad == kFastNotStaged ? 0u : pad * 16u;
  r.a = __uint_as_float(uniform(A[2]));
  r.s = __uint_as_float(uniform(A[3]));
  const uint32_t b0 = uniform(B[0]);
  r.dt = (b0 >> 16) & 0xff;
  r.s1 = b0 >> 24;
  r.base = uniform(B[1]) & 0xffff;
  r.off = (int32_t)uniform(B[2]);
  r.s0 = (int32_t)uniform(B[3]);
  return r;
}

// Copy the staged views' chunks (every loaded view with column stride 1)
// into the arena, each lane its own chunks (chunk q at staged + 16 q; an fp32
// view's second plane follows at + 16 * G * kBlock).  Issued before the main
// loop, so the loads are in flight under it.  Returns false (uniform) when a
// view's base is not 16-byte aligned: the batches then run the epilogue.
template <int G>
DEV bool fast_prefetch(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t ins_off, const ItemState& st) {
  FastChunks<G> c;
  fast_chunks<G>(tid, t, st, c);
  const uint32_t wave = uniform(tid / 64);
  const uint32_t lds = (uint32_t)(uintptr_t)(LDS uint8_t*)g_smem;
  constexpr uint32_t kPlane = 16u * G * kBlock;
  bool ok = true;
  const uint32_t n = t.expr_len;
  // the next record's words are read while this one is handled
  u32x4 cA = {0, 0, 0, 0}, cB = {0, 0, 0, 0};
  if (n > 0) {
    cA = frec_word(ins_off, t.fin_first);
    cB = frec_word(ins_off, t.fin_first + 1);
  }
  for (uint32_t pc = 0; pc < n; ++pc) {
    const uint32_t nx = t.fin_first + 2 * (pc + 1 < n ? pc + 1 : pc);
    const u32x4 nA = frec_word(ins_off, nx), nB = frec_word(ins_off, nx + 1);
    const FRec r = frec_decode(cA, cB);
    cA = nA;
    cB = nB;
    const uint32_t op = r.w0 & 0xff, src = (r.w0 >> 8) & 0xff;
    if (op != VM_STORE && src != SRC_VIEW) continue;
    const GLOBAL uint8_t* p = base_ptr(ka, r.base < (uint32_t)kMaxBases ? r.base : 0u);
    if (r.s1 == 1 && ((uintptr_t)p & 15) != 0) ok = false;
    if (!r.staged || !ok) continue;
    const uint32_t es = r.dt == DT_F32 ? 4u : 2u;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t idx = c.ok[g] ? r.off + c.row[g] * r.s0 + c.col[g] : r.off;
      const GLOBAL uint8_t* gp = p + (int64_t)idx * es;
      const uint32_t m0 = lds + r.staged + 16u * (uint32_t)(g * kBlock) + 1024u * wave;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gp), "s"(m0) : "m0");
      if (r.dt == DT_F32) {
        const GLOBAL uint8_t* gp2 = gp + 16;
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gp2), "s"(m0 + kPlane) : "m0");
      }
    }
  }
  return ok;
}

// A view with column stride 0: one element per chunk, broadcast along the
// chunk (the dtype branch taken once, outside the chunk loops).
template <int G>
DEV void fast_load_bcast(const GLOBAL uint8_t* p, uint32_t dt, const int32_t (&idx)[G], float (&x)[G][8]) {
  float e[G];
  if (dt == DT_F32) {
#pragma unroll
    for (int g = 0; g < G; ++g) e[g] = ((const GLOBAL float*)p)[idx[g]];
  } else {
    const GLOBAL uint16_t* q = (const GLOBAL uint16_t*)p;
    uint32_t h[G];
#pragma unroll
    for (int g = 0; g < G; ++g) h[g] = q[idx[g]];
    if (dt == DT_BF16) {
#pragma unroll
      for (int g = 0; g < G; ++g) e[g] = bf16_bits_to_f32(h[g]);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) e[g] = f16_bits_to_f32(h[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[g][j] = e[g];
}

// Stores of the chunks in bounds, converted to the view's dtype (RNE), as
// store_chunks.
template <int G>
DEV void fast_store(GLOBAL uint8_t* p, uint32_t dt, const int32_t (&idx)[G], const bool (&ok)[G],
                    const float (&y)[G][8]) {
  if (dt == DT_F32) {
    GLOBAL float* q = (GLOBAL float*)p;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g]) continue;
      u32x4 r0, r1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r0[j] = __float_as_uint(y[g][j]);
        r1[j] = __float_as_uint(y[g][4 + j]);
      }
      *(GLOBAL u32x4*)(q + idx[g]) = r0;
      *(GLOBAL u32x4*)(q + idx[g] + 4) = r1;
    }
  } else if (dt == DT_BF16) {
    GLOBAL uint16_t* q = (GLOBAL uint16_t*)p;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g]) continue;
      u32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = narrow2<true>(y[g][2 * j], y[g][2 * j + 1]);
      *(GLOBAL u32x4*)(q + idx[g]) = r;
    }
  } else {
    GLOBAL uint16_t* q = (GLOBAL uint16_t*)p;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g]) continue;
      u32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = narrow2<false>(y[g][2 * j], y[g][2 * j + 1]);
      *(GLOBAL u32x4*)(q + idx[g]) = r;
    }
  }
}

// Run the program over this thread's G chunks (fast_prefetch staged the
// loads of its unit-stride views).  The record of instruction pc + 1 is read
// while instruction pc runs.
template <int G>
DEV void fast_run(uint32_t tid, const Ctx& ka, const DTask& t, uint32_t ins_off, const ItemState& st) {
  wait_vmcnt<0>();  // this lane's staged chunks have landed in LDS
  asm volatile("" ::: "memory");
  constexpr uint32_t kPlane = 16u * G * kBlock;
  FastChunks<G> c;
  fast_chunks<G>(tid, t, st, c);
  const int pitch = st.bn + 4;
  const LDS float* ctile = (const LDS float*)g_smem;
  float y[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    // rows are 16-byte aligned (pitch a multiple of 4), chunks start at multiples of 8
    const LDS float* src = ctile + c.r[g] * pitch + c.cc[g];
    const u32x4 lo = *(const LDS u32x4*)src, hi = *(const LDS u32x4*)(src + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[g][j] = __uint_as_float(lo[j]);
      y[g][4 + j] = __uint_as_float(hi[j]);
    }
  }
  const uint32_t n = t.expr_len;
  FRec r = frec_decode(frec_word(ins_off, t.fin_first), frec_word(ins_off, t.fin_first + 1));
#pragma nounroll
  for (uint32_t pc = 0; pc < n; ++pc) {
    // the next record's words (clamped to the program), in flight while this one runs
    const uint32_t nx = t.fin_first + 2 * (pc + 1 < n ? pc + 1 : pc);
    const u32x4 nA = frec_word(ins_off, nx), nB = frec_word(ins_off, nx + 1);
    const uint32_t op = r.w0 & 0xff, src = (r.w0 >> 8) & 0xff, rnd = (r.w0 >> 16) & 0xff, rev = r.w0 >> 24;
    const float a = r.a;
    float x[G][8];
    if (op == VM_STORE) {
      GLOBAL uint8_t* p = base_ptr(ka, r.base < (uint32_t)kMaxBases ? r.base : 0u);
      int32_t idx[G];
#pragma unroll
      for (int g = 0; g < G; ++g) idx[g] = c.ok[g] ? r.off + c.row[g] * r.s0 + c.col[g] : r.off;
      fast_store<G>(p, r.dt, idx, c.ok, y);
      r = frec_decode(nA, nB);
      continue;
    }
    if (src == SRC_VIEW) {
      if (r.staged) {
        // this lane's chunk g of the view sits at staged + 16 (g * kBlock + tid)
        const LDS uint8_t* base = (const LDS uint8_t*)(g_smem + r.staged + 16u * tid);
        if (r.dt == DT_F32) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const u32x4 v = *(const LDS u32x4*)(base + 16u * g * kBlock);
            const u32x4 v2 = *(const LDS u32x4*)(base + kPlane + 16u * g * kBlock);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[g][j] = __uint_as_float(v[j]);
              x[g][4 + j] = __uint_as_float(v2[j]);
            }
          }
        } else if (r.dt == DT_BF16) {
#pragma unroll
          for (int g = 0; g < G; ++g) widen8<true>(*(const LDS u32x4*)(base + 16u * g * kBlock), x[g]);
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) widen8<false>(*(const LDS u32x4*)(base + 16u * g * kBlock), x[g]);
        }
      } else {
        // column stride 0: one element per chunk, broadcast along the chunk
        const GLOBAL uint8_t* p = base_ptr(ka, r.base < (uint32_t)kMaxBases ? r.base : 0u);
        int32_t idx[G];
#pragma unroll
        for (int g = 0; g < G; ++g) idx[g] = c.ok[g] ? r.off + c.row[g] * r.s0 : r.off;
        fast_load_bcast<G>(p, r.dt, idx, x);
      }
    } else {
      const float k = src == SRC_SCALAR ? r.s : 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[g][j] = k;
    }
#define TK_EACH_R(expr)                          \
  _Pragma("unroll") for (int g = 0; g < G; ++g)  \
  _Pragma("unroll") for (int j = 0; j < 8; ++j) { \
    float& v = y[g][j];                          \
    const float o = x[g][j];                     \
    (void)o;                                     \
    expr;                                        \
  }
    switch (op) {
      case VM_LOAD: TK_EACH_R(v = o) break;
      case VM_ADD:
        if (rev) { TK_EACH_R(float u = a * v; v = o + u) }
        else { TK_EACH_R(float u = a * o; v = v + u) }
        break;
      case VM_SUB:
        if (rev) { TK_EACH_R(float u = a * v; v = o - u) }
        else { TK_EACH_R(float u = a * o; v = v - u) }
        break;
      case VM_MUL: TK_EACH_R(v = v * o) break;
      case VM_DIV:
        if (rev) { TK_EACH_R(v = o / v) }
        else { TK_EACH_R(v = v / o) }
        break;
      case VM_NEG: TK_EACH_R(v = -v) break;
      case VM_RELU: TK_EACH_R(v = v < 0.0f ? 0.0f : v) break;
      case VM_SQUARE: TK_EACH_R(v = v * v) break;
      case VM_TB:
        if (rev) { TK_EACH_R(v = v <= a ? 0.0f : o) }
        else { TK_EACH_R(v = o <= a ? 0.0f : v) }
        break;
      case VM_SCALE: TK_EACH_R(v = a * v) break;
      case VM_ZERO: TK_EACH_R(v = 0.0f) break;
      default: break;
    }
#undef TK_EACH_R
    if (rnd == DT_BF16) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) y[g][j] = bf16_bits_to_f32(f32_to_bf16_bits(y[g][j]));
    } else if (rnd == DT_F16) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) y[g][j] = f16_bits_to_f32(f32_to_f16_bits(y[g][j]));
    }
    r = frec_decode(nA, nB);
  }
}

// Geometry of a direct column reduction's item: CC column chunks of 8 by
// 256 / CC row lanes (32 x 8, or 8 x 32 with F_COLLANES32).
DEV uint32_t col_chunks(const DTask& t) { return (t.flags & F_COLLANES32) ? 8u : 32u; }

// A column reduction whose source program is one load of a 2-D view with
// column stride 1 (F_COLDIRECT): thread (row lane rl = tid / CC, chunk
// cc = tid % CC) sums rows rb + rl, rb + rl + RL, ... of its 8 columns
// straight from memory, 16 rows in flight at a time, into its running sums
// (with 32 chunks by 8 lanes the rows and additions come in the order the
// batches would take them, so the sums are bit-identical to theirs).
template <uint32_t CC>
DEV void red_cols_direct(uint32_t tid, const Ctx& ka, const DTask& t, const DStage& sd, uint32_t item,
                         ItemState& st) {
  const uint32_t cb = item / t.split, part = item % t.split;
  const uint32_t cols = t.m, R = t.k;
  constexpr uint32_t RL = kBlock / CC;
  const uint32_t cc = tid % CC, rl = tid / CC;
  const uint32_t col = cb * CC * 8 + cc * 8;
  const uint32_t rb = part * t.kchunk;
  const uint32_t re = (rb + t.kchunk < R) ? rb + t.kchunk : R;
  const LDS uint32_t* iw = (const LDS uint32_t*)(g_plan + sd.off_ins + t.expr_first * sizeof(DIns));
  const VView v = load_view(sd.off_views + (uniform(iw[1]) & 0xffff) * sizeof(DView));
  const GLOBAL uint8_t* p = base_ptr(ka, v.base);
  const uint32_t dt = v.dtype;
  const int32_t epc = dt == DT_F32 ? 4 : 8;
  const bool vec = aligned16(p) && v.offset % epc == 0 && v.stride[0] % epc == 0;
  if (col >= cols || rb >= re) return;
  constexpr int U = 16;
  for (uint32_t r0 = rb + rl; r0 < re; r0 += RL * U) {
    float x[U][8];
    int32_t idx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t r = r0 + RL * u;
      idx[u] = v.offset + (int32_t)(r < re ? r : rb) * v.stride[0] + (int32_t)col;
    }
    if (dt == DT_F32) {
      const GLOBAL float* q = (const GLOBAL float*)p;
      if (vec) {
        u32x4 a[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          a[u][0] = *(const GLOBAL u32x4*)(q + idx[u]);
          a[u][1] = *(const GLOBAL u32x4*)(q + idx[u] + 4);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) x[u][j] = __uint_as_float(a[u][j / 4][j % 4]);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) x[u][j] = q[idx[u] + j];
      }
    } else {
      const GLOBAL uint16_t* q = (const GLOBAL uint16_t*)p;
      const bool bf = dt == DT_BF16;
      if (vec) {
        u32x4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = *(const GLOBAL u32x4*)(q + idx[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            x[u][j] = half_bits_to_f32((j & 1) ? a[u][j / 2] >> 16 : a[u][j / 2] & 0xffffu, bf);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) x[u][j] = half_bits_to_f32(q[idx[u] + j], bf);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (r0 + RL * u < re)
#pragma unroll
        for (int j = 0; j < 8; ++j) st.acc8[j] = st.acc8[j] + x[u][j];
  }
}

// Finish of a directly read column sum: after red_cols_direct each thread
// holds the sums of its 8 columns over its row lane's rows.  The RL row lanes
// are combined through LDS in order (lane 0 first); then thread i < 8 CC
// takes column cb * 8 CC + i and writes its part's partial (F_PARTIAL) or
// runs the finishing program for it (operands preloaded before the sums).
template <uint32_t CC>
DEV void red_cols_finish(uint32_t tid, const Ctx& ka, const DTask& t, const DStage& sd, uint32_t item,
                         const ItemState& st, const uint32_t (&raw)[kPre], uint32_t npre) {
  const uint32_t cb = item / t.split, part = item % t.split;
  const uint32_t cols = t.m;
  constexpr uint32_t RL = kBlock / CC, W = CC * 8;
  const uint32_t cc = tid % CC, rl = tid / CC;
  LDS float* red = (LDS float*)g_smem;  // [RL row lanes][8 CC columns]
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rl * W + cc * 8 + j] = st.acc8[j];
  __syncthreads();
  if (tid >= W) return;
  const uint32_t col = cb * W + tid;
  float a = red[tid];
#pragma unroll
  for (uint32_t q = 1; q < RL; ++q) a = a + red[q * W + tid];
  const bool ok = col < cols;
  if (t.flags & F_PARTIAL) {
    if (ok) ws_f32(ka, t.scratch)[(uint64_t)part * cols + col] = a;
    return;
  }
  const uint32_t c[kMaxDims] = {ok ? col : 0u, 0u, 0u, 0u};
  prog_run(tid, ka, sd.off_views, sd.off_ins + t.fin_first * sizeof(DIns), t.fin_len, c, ok, a, raw, npre);
}

// A column reduction read directly: its finishing program's leading operands
// are loaded first, then the rows, then the finish.
DEV void red_cols_item(uint32_t tid, const Ctx& ka, const DTask& t, const DStage& sd, uint32_t item, ItemState& st) {
  uint32_t raw[kPre] = {0, 0, 0, 0};
  uint32_t npre = 0;
  if (!(t.flags & F_PARTIAL)) {
    const uint32_t col = (item / t.split) * col_chunks(t) * 8 + tid;
    const uint32_t c[kMaxDims] = {col < t.m ? col : 0u, 0u, 0u, 0u};
    npre = prog_preload(ka, sd.off_views, sd.off_ins + t.fin_first * sizeof(DIns), t.fin_len, c, raw);
  }
  if (t.flags & F_COLLANES32) {
    red_cols_direct<8>(tid, ka, t, sd, item, st);
    red_cols_finish<8>(tid, ka, t, sd, item, st, raw, npre);
  } else {
    red_cols_direct<32>(tid, ka, t, sd, item, st);
    red_cols_finish<32>(tid, ka, t, sd, item, st, raw, npre);
  }
}

// Combine of a two-phase reduction's partials.  Default: one thread per
// output, its parts summed in order with sixteen loads in flight.  F_ROWWG
// (few outputs, many parts): output `item`, thread t sums parts t, t + 256,
// ... in order, then a fixed-order block sum.  Then the finishing program,
// its leading operands preloaded before the partials.
DEV void red_final_item(uint32_t tid, const Ctx& ka, const DTask& t, const DStage& sd, uint32_t item) {
  const GLOBAL float* P = ws_f32(ka, t.scratch);
  const bool cols_layout = (t.tile & 1) != 0;  // [parts][rows] instead of [rows][parts]
  const uint32_t fin = sd.off_ins + t.fin_first * sizeof(DIns);
  const bool rowwg = (t.flags & F_ROWWG) != 0;
  const uint32_t row = rowwg ? item : item * kBlock + tid;
  const bool exists = row < t.m;
  const uint32_t c[kMaxDims] = {exists ? row : 0u, 0u, 0u, 0u};
  uint32_t raw[kPre] = {0, 0, 0, 0};
  const uint32_t npre = prog_preload(ka, sd.off_views, fin, t.fin_len, c, raw);
  float a = 0.0f;
  if (rowwg) {
    for (uint32_t p = tid; p < t.split; p += kBlock)
      a = a + (cols_layout ? P[(uint64_t)p * t.m + row] : P[(uint64_t)row * t.split + p]);
    a = block_sum(tid, a);
  } else {
    const uint32_t rr = exists ? row : 0u;
    for (uint32_t p0 = 0; p0 < t.split; p0 += 16) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t pp = p0 + i < t.split ? p0 + i : 0u;
        v[i] = cols_layout ? P[(uint64_t)pp * t.m + rr] : P[(uint64_t)rr * t.split + pp];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (p0 + i < t.split) a = a + v[i];
    }
  }
  prog_run(tid, ka, sd.off_views, fin, t.fin_len, c, exists && (!rowwg || tid == 0), a, raw, npre);
}

// Column sums of a contraction's B operand over all of K, by the tiles of
// the first tile row (F_BSUM): a column reduction of the same 2-D value B
// reads runs here instead of as items of its own.  Where the main loop
// summed B's fragments (gemm_mfma's direct path), the two halves per column
// come from the C tile's padding.  Otherwise the tile reads B again: thread
// (row lane rl, chunk cc) sums rows rl, rl + RL, ... of 8 columns of the
// tile's column block, 16 rows in flight (CC x RL = 16 x 16 for 128-wide
// tiles, 8 x 32 for 64-wide), and the row lanes are combined through LDS in
// order.  Then thread i < bn runs the reduction's finishing program for
// column n0 + i, its leading operands loaded before the sums.
template <bool BF>
DEV void bsum_rows(const GLOBAL uint16_t* p, const VView& B, uint32_t K, uint32_t N, uint32_t col, uint32_t rl,
                   uint32_t RL, bool vec, float (&acc)[8]) {
  constexpr int U = 16;
  for (uint32_t r0 = rl; r0 < K; r0 += RL * U) {
    if (vec) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + RL * u < K ? r0 + RL * u : 0u;
        v[u] = *(const GLOBAL u32x4*)(p + B.offset + (int64_t)r * B.stride[0] + col);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r0 + RL * u >= K) continue;
        float x[8];
        widen8<BF>(v[u], x);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = acc[j] + x[j];
      }
    } else {
      for (int u = 0; u < U; ++u) {
        const uint32_t r = r0 + RL * u;
        if (r >= K) break;
        for (int j = 0; j < 8; ++j)
          if (col + j < N)
            acc[j] = acc[j] + half_bits_to_f32(p[B.offset + (int64_t)r * B.stride[0] + (int64_t)(col + j) * B.stride[1]], BF);
      }
    }
  }
}

DEV void bsum_tile(uint32_t tid, const Ctx& ka, const DTask& t, const DStage& sd, const ItemState& st, bool summed) {
  if (st.m0 != 0) return;
  // B's element (n, k) at off + k * stride[0] + n * stride[1]
  const VView B = load_view(sd.off_views + t.vb * sizeof(DView));
  const GLOBAL uint16_t* p = (const GLOBAL uint16_t*)base_ptr(ka, B.base);
  const uint32_t bn = st.bn, n0 = st.n0, K = t.k, N = t.n;
  const uint32_t CC = bn / 8, RL = kBlock / CC;
  const uint32_t cc = tid % CC, rl = tid / CC;
  const uint32_t col = n0 + cc * 8;
  const uint32_t fin = sd.off_ins + t.bs_first * sizeof(DIns);
  const uint32_t me = n0 + tid;
  const uint32_t c[kMaxDims] = {me < N ? me : 0u, 0u, 0u, 0u};
  uint32_t raw[kPre] = {0, 0, 0, 0};
  const uint32_t npre = tid < bn ? prog_preload(ka, sd.off_views, fin, t.bs_len, c, raw) : 0u;
  if (summed) {
    // the main loop's sums, two halves per column in the C tile's padding
    if (tid < bn) {
      const LDS float* pad = (const LDS float*)g_smem + bn;
      const uint32_t pitch = bn + 4, p = 2 * tid;
      const float a = pad[(p / 4) * pitch + p % 4] + pad[((p + 1) / 4) * pitch + (p + 1) % 4];
      prog_run(tid, ka, sd.off_views, fin, t.bs_len, c, me < N, a, raw, npre);
    }
    __syncthreads();  // the next item may overwrite the tile and the slots
    return;
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  if (col < N) {
    const bool vec = aligned16(p) && B.stride[1] == 1 && N % 8 == 0 && (B.offset & 7) == 0 && (B.stride[0] & 7) == 0;
    if (B.dtype == DT_BF16)
      bsum_rows<true>(p, B, K, N, col, rl, RL, vec, acc);
    else
      bsum_rows<false>(p, B, K, N, col, rl, RL, vec, acc);
  }
  LDS float* red = (LDS float*)g_smem;  // [RL row lanes][bn columns]
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rl * bn + cc * 8 + j] = acc[j];
  __syncthreads();
  if (tid < bn) {
    float a = red[tid];
    for (uint32_t q = 1; q < RL; ++q) a = a + red[q * bn + tid];
    prog_run(tid, ka, sd.off_views, fin, t.bs_len, c, me < N, a, raw, npre);
  }
  __syncthreads();  // the next item may overwrite the LDS sums and the slots
}

// A stage record from the plan (wave-uniform).
DEV DStage load_stage(const GLOBAL uint8_t* stages, uint32_t s) {
  constexpr int N = sizeof(DStage) / 4;
  const GLOBAL uint32_t* w = (const GLOBAL uint32_t*)(stages + s * sizeof(DStage));
  struct Words {
    uint32_t u[N];
  } r;
#pragma unroll
  for (int k = 0; k < N; ++k) r.u[k] = uniform(w[k]);
  return __builtin_bit_cast(DStage, r);
}

// One work item: prologue, then batches through the machine.
DEV void run_item(const Ctx& ka, const DTask& t, const DStage& sd, uint32_t item) {
  // The thread index passes through an empty asm once per item, so values
  // derived from it (LDS addresses, tile offsets) are computed per item
  // instead of being hoisted out of the stage loop and held in registers
  // for the whole launch.
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  ItemState st;
  st.m0 = st.n0 = st.split_index = 0;
  st.bm = st.bn = 0;
  st.acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.acc8[j] = 0.0f;
  switch (t.kind) {
    case T_GEMM_SIMT:
      gemm_simt(tid, ka, t, sd.off_views, item, st);
      __syncthreads();
      if (t.flags & F_FASTEPI) {
        if (fast_prefetch<2>(tid, ka, t, sd.off_ins, st)) {
          fast_run<2>(tid, ka, t, sd.off_ins, st);
          __syncthreads();  // the next item may overwrite the LDS tile and the prefetched operands
          return;
        }
        wait_vmcnt<0>();  // staged loads may still be writing the slots the batches use
      }
      break;
    case T_GEMM_MFMA: {
      // the operand dtype is the A view's (both operands share it)
      const bool bf16 = uniform(((const LDS DView*)(g_plan + sd.off_views + t.va * sizeof(DView)))->dtype) == DT_BF16;
      // a register epilogue's operands are fetched into LDS under the main loop
      bool fast = false;
      auto before_loop = [&]() {
        if (!(t.flags & F_FASTEPI)) return;
        fast = t.tile == 0 ? fast_prefetch<8>(tid, ka, t, sd.off_ins, st) : fast_prefetch<2>(tid, ka, t, sd.off_ins, st);
      };
      bool csum;
      if (t.tile == 0) {
        if (bf16)
          csum = gemm_mfma<128, 128, true>(tid, ka, t, sd.off_views, item, st, before_loop);
        else
          csum = gemm_mfma<128, 128, false>(tid, ka, t, sd.off_views, item, st, before_loop);
      } else {
        if (bf16)
          csum = gemm_mfma<64, 64, true>(tid, ka, t, sd.off_views, item, st, before_loop);
        else
          csum = gemm_mfma<64, 64, false>(tid, ka, t, sd.off_views, item, st, before_loop);
      }
      __syncthreads();
      if (fast) {
        if (t.tile == 0)
          fast_run<8>(tid, ka, t, sd.off_ins, st);
        else
          fast_run<2>(tid, ka, t, sd.off_ins, st);
        __syncthreads();  // the next item may overwrite the LDS tile and the prefetched operands
        if (t.flags & F_BSUM) bsum_tile(tid, ka, t, sd, st, csum);
        return;
      }
      // a misaligned operand: the batches run the epilogue, over slots the
      // staged loads may still be writing
      if (t.flags & F_FASTEPI) wait_vmcnt<0>();
      break;
    }
    case T_GEMV_Q8: {
      uint32_t raw[kPre] = {0, 0, 0, 0};
      const uint32_t npre = gemv_epi_preload(tid, ka, t, sd.off_views, sd.off_ins, item, raw);
      gemv_q8(tid, ka, t, sd.off_views, item);
      gemv_epilogue(tid, ka, t, sd.off_views, sd.off_ins, item, raw, npre);
      __syncthreads();  // the next item may overwrite the row sums and the slots
      return;
    }
    case T_RED_COLS:
      if (t.flags & F_COLDIRECT) {
        red_cols_item(tid, ka, t, sd, item, st);
        __syncthreads();  // the next item may overwrite the LDS sums and the slots
        return;
      }
      break;
    case T_RED_FINAL:
      red_final_item(tid, ka, t, sd, item);
      __syncthreads();  // the next item may overwrite the LDS sums and the slots
      return;
    default:
      break;
  }
  trace_stamp(ka, 0x300);
  for (uint32_t bi = 0;; ++bi) {
    Batch b;
    uint32_t live;
    if (!fill(tid, ka, t, sd.off_ins, item, bi, st, b, live)) break;
    if (live) {
      if (b.width == 8)
        vm_run<8, 2>(tid, ka, b, sd.off_views, live);
      else
        vm_run<1, 16>(tid, ka, b, sd.off_views, live);
    }
    consume(tid, t, b, live, st);
    trace_stamp(ka, 0x400 + bi);
  }
  // the next item may overwrite the LDS tile and scratch
  __syncthreads();
  // (the batches may have overwritten the sums in the tile's padding)
  if (t.kind == T_GEMM_MFMA && (t.flags & F_BSUM)) bsum_tile(tid, ka, t, sd, st, false);
}

// Grid barrier: every workgroup gathers every arrival itself.
//
// Arrival: thread 0 of each workgroup releases its writes (agent-scope fence)
// and stores the epoch into its own arrival flag (one u32 per workgroup, the
// flags packed 16 to a 64-byte line).  Then the first wave of every workgroup
// polls all arrival flags (4 per lane, in flight together) until each holds
// at least the epoch, and acquires (agent-scope fence).  With no release flag
// written by a gathering workgroup, the last arrival reaches every workgroup
// after one store and one poll instead of two of each.  Epochs grow
// monotonically across launches on a workspace (the base is kept in the
// header), so flags never need resetting.  Every spin is bounded by the
// deadline; a timeout sets the abort word, which every spinner also watches.
// next(copy) runs once every wave is past its last read of the current
// stage's descriptors: in wave 0 after the arrival, under the polls (copy
// false), and in waves 1-3 while wave 0 polls (copy true: they also copy the
// next stage's descriptors into LDS); the plan never changes during a launch,
// so those reads need no ordering against the barrier.
template <class Next>
DEV bool grid_barrier(const Ctx& ka, uint32_t epoch, uint32_t stage, uint64_t deadline, Next next) {
  __shared__ uint32_t s_ok;
  GLOBAL uint32_t* arrive = (GLOBAL uint32_t*)(ka.ws + kHdrArrive);
  GLOBAL uint32_t* abort = (GLOBAL uint32_t*)(ka.ws + kHdrAbort);
  const uint32_t G = gridDim.x, bid = blockIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(arrive + bid, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < 64) {
    next(false);
    uint32_t ok = 1;
    const uint32_t lane = threadIdx.x;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t base = 0; base < G; base += 256) {
      GLOBAL uint32_t* f[4];
      bool live[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = base + lane + 64 * i;
        live[i] = w < G;
        f[i] = arrive + (live[i] ? w : 0);
      }
      for (;;) {
        bool done = true;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (live[i]) {
            const uint32_t v = __hip_atomic_load(f[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((int32_t)(v - epoch) < 0) done = false;
          }
        if (__all(done)) break;
        if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          ok = 0;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > deadline) {
          set_abort(ka, stage);
          ok = 0;
          break;
        }
      }
      if (!ok) break;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const uint32_t all_ok = __builtin_amdgcn_readfirstlane(ok) & (uint32_t)__all(ok);
    if (lane == 0) s_ok = all_ok;
  } else {
    next(true);
  }
  __syncthreads();
  return s_ok != 0;
}

DEV uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Copy a stage blob into LDS (threads first .. kBlock - 1; 16-byte chunks).
// The scheduler keeps every stage blob within kPlanLds bytes.
DEV void stage_blob_to_lds(const GLOBAL uint8_t* plan, const DStage& st, uint32_t first) {
  const GLOBAL u32x4* src = (const GLOBAL u32x4*)(plan + st.blob_off);
  LDS u32x4* dst = (LDS u32x4*)g_plan;
  const uint32_t n = (st.blob_bytes < kPlanLds ? st.blob_bytes : kPlanLds) / 16;
  for (uint32_t i = threadIdx.x - first; i < n; i += kBlock - first) dst[i] = src[i];
}

// A stage record assigned in divergent-looking code, made wave-uniform again.
DEV DStage uniform_stage(const DStage& sd) {
  constexpr int N = sizeof(DStage) / 4;
  struct Words {
    uint32_t u[N];
  } r = __builtin_bit_cast(Words, sd);
#pragma unroll
  for (int k = 0; k < N; ++k) r.u[k] = uniform(r.u[k]);
  return __builtin_bit_cast(DStage, r);
}

}  // namespace

__global__ __launch_bounds__(kBlock, 1) void tk_persistent(KArgs) {
  // The argument block stays in the kernel argument segment (read in place, so
  // the base table is never copied into private memory); it is read once here.
  const KArgs& kargs = *(const KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  Ctx ka;
  ka.ws = (GLOBAL uint8_t*)uniform64((int64_t)kargs.ws);
  ka.plan = (const GLOBAL uint8_t*)uniform64((int64_t)kargs.plan);
  ka.flags = uniform(kargs.flags);
  ka.stagger_seed = uniform(kargs.stagger_seed);
  ka.host_abort = (uint32_t*)uniform64((int64_t)kargs.host_abort);
  const uint32_t n_bases = kargs.n_bases < (uint32_t)kMaxBases ? kargs.n_bases : (uint32_t)kMaxBases;
  for (uint32_t i = threadIdx.x; i < n_bases; i += kBlock) ((LDS uint64_t*)g_bases)[i] = (uint64_t)kargs.bases[i];
  const uint64_t deadline = kargs.deadline_ticks ? kargs.deadline_ticks : 400000000ull;  // 4 s at 100 MHz
  const GLOBAL DHeader* h = (const GLOBAL DHeader*)ka.plan;
  const GLOBAL uint8_t* stages = ka.plan + h->off_stages;
  const uint32_t n_stages = h->n_stages;
  if (*(volatile GLOBAL uint32_t*)(ka.ws + kHdrAbort) != 0u) {
    // a previous launch on this workspace stopped: run nothing, and say so
    // to the host again (its words may have been cleared for another workspace)
    if (blockIdx.x == 0 && threadIdx.x == 0 && ka.host_abort) {
      __hip_atomic_store(ka.host_abort + 1, *(volatile GLOBAL uint32_t*)(ka.ws + kHdrAbortStage), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(ka.host_abort, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  const uint32_t epoch0 = *(volatile GLOBAL uint32_t*)(ka.ws + kHdrEpoch);
  if (n_stages == 0) return;
  DStage sd = load_stage(stages, 0);
  stage_blob_to_lds(ka.plan, sd, 0);
  __syncthreads();
  if ((ka.flags & K_TIMESTAMPS) && blockIdx.x == 0 && threadIdx.x == 0)
    ((GLOBAL uint64_t*)(ka.ws + kHdrStamps))[0] = __builtin_amdgcn_s_memrealtime();
  trace_stamp(ka, 0xffffffffu);
  for (uint32_t s = 0; s < n_stages; ++s) {
    uint32_t ti = 0;
    for (uint32_t item = blockIdx.x; item < sd.n_items; item += gridDim.x) {
      while (ti + 1 < sd.n_tasks && item >= task_item_begin(ti + 1)) ++ti;
      const DTask t = load_task(ti);
      if (ka.flags & K_STAGGER) {
        uint32_t n = hash32(ka.stagger_seed ^ (blockIdx.x * 0x9e3779b9u) ^ (item * 0x85ebca6bu) ^ s) % 48u;
        for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
      }
      trace_stamp(ka, 0x1000 + s);
      run_item(ka, t, sd, item - t.item_begin);
      trace_stamp(ka, 0x2000 + s);
    }
    if (s + 1 < n_stages) {
      const bool stamp = (ka.flags & K_TIMESTAMPS) && blockIdx.x == 0 && threadIdx.x == 0 && s < kMaxTimedStages;
      GLOBAL uint64_t* stamps = (GLOBAL uint64_t*)(ka.ws + kHdrStamps) + 4 * s;
      if (stamp) {
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        stamps[1] = now;
        stamps[2] = now;  // (the next stage's descriptors are staged inside the barrier)
      }
      // the next stage's descriptors are read and staged while the barrier
      // completes, off the path from the last item to the arrival
      const bool ok = grid_barrier(ka, epoch0 + s + 1, s, deadline, [&](bool copy) {
        sd = load_stage(stages, s + 1);
        if (copy) stage_blob_to_lds(ka.plan, sd, 64);
      });
      if (!ok) return;
      sd = uniform_stage(sd);
      if (stamp) stamps[3] = __builtin_amdgcn_s_memrealtime();
      if (stamp && s + 1 < kMaxTimedStages) stamps[4] = stamps[3];
    }
  }
  // The next launch on this workspace continues the epoch sequence.  Every
  // workgroup has read the base before the first barrier, which this
  // workgroup has passed.
  if (n_stages > 1 && blockIdx.x == 0 && threadIdx.x == 0)
    *(volatile GLOBAL uint32_t*)(ka.ws + kHdrEpoch) = epoch0 + n_stages - 1;
}

__global__ void tk_zero_header(uint8_t* ws, uint32_t bytes) {
  for (uint32_t i = threadIdx.x * 4; i < bytes; i += blockDim.x * 4) *(uint32_t*)(ws + i) = 0u;
}

// The workspace of tk_run_into_noalloc, for callers that cannot allocate:
// one copy per device, in the code object's own memory, held until the
// process ends.  Host code never uses this name as an address (on the host
// it is a stand-in, not device memory): tk_device_static_workspace looks up
// each device's copy once, with that device current, and every launch and
// fill takes that pointer.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t tk_device_static_workspace(int device, void** out) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* ptrs[kDevices] = {};
  if (device < 0 || device >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[device] = p;
  }
  *out = ptrs[device];
  return hipSuccess;
}

// Host-side launch helpers used by the C ABI.
hipError_t tk_device_launch(const KArgs& ka, int grid, hipStream_t stream) {
  void* args[] = {(void*)&ka};
  return hipLaunchCooperativeKernel((const void*)tk_persistent, dim3(grid), dim3(kBlock), args, 0, stream);
}

// Ordinary launch of a grid the compiler sized to be co-resident (occupancy x
// CUs); the barrier's bounded wait covers a device shared with other work.
hipError_t tk_device_launch_resident(const KArgs& ka, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(tk_persistent, dim3(grid), dim3(kBlock), 0, stream, ka);
  return hipGetLastError();
}

hipError_t tk_device_occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)tk_persistent, kBlock, 0);
}

hipError_t tk_device_attributes(hipFuncAttributes* attr) {
  return hipFuncGetAttributes(attr, (const void*)tk_persistent);
}

hipError_t tk_device_zero_header(uint8_t* ws, hipStream_t stream) {
  hipLaunchKernelGGL(tk_zero_header, dim3(1), dim3(256), 0, stream, ws, kHeaderBytes);
  return hipGetLastError();
}
