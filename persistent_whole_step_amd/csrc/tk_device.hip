// The persistent whole-step kernel for gfx950 (MI355X).
//
// One cooperative launch runs a whole compiled program: every workgroup walks
// the plan's stages, takes the stage's work items round-robin
// (item = blockIdx.x + i * gridDim.x), and all workgroups meet at a
// global-memory grid barrier between stages.  This is the execution model of
// the trainkernel generator (codegen.py `_Generator.generate`: operators in
// topological order separated by `mk_grid_sync`; the device helpers of
// `_CUDA_PREAMBLE`), re-designed as an interpreter of a device-resident plan:
//   * pointwise work and every epilogue run on a small accumulator machine over
//     chunks of 8 consecutive elements per lane (vector loads/stores);
//   * contractions with bf16/f16 operands run on MFMA 32x32x16 tiles with
//     LDS double buffering; other dtypes use an fp32-FMA tile whose per-output
//     accumulation is sequential in k;
//   * one-row int8-weight products stream the weight once, split along K over
//     the 64 lanes of a wave;
//   * reductions sum fixed partitions in a fixed order (deterministic, every
//     element covered).
// Built with -ffp-contract=off: no implicit fused multiply-adds, so pointwise
// results equal IEEE binary32 step by step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

using namespace tkplan;

#define DEV __device__ __forceinline__

namespace {

constexpr int kSmemBytes = 2 * 2 * 128 * 72 * 2;  // A and B tiles, double buffered (73728 B)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ conversions --

DEV float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 with round-to-nearest-even; NaN stays a quiet NaN.
DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

DEV float f16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

DEV uint32_t f32_to_f16_bits(float f) {
  _Float16 v = (_Float16)f;  // v_cvt_f16_f32: round-to-nearest-even, subnormals kept
  return (uint32_t)__builtin_bit_cast(uint16_t, v);
}

DEV float round_to(float x, uint32_t dt) {
  if (dt == DT_BF16) return bf16_bits_to_f32(f32_to_bf16_bits(x));
  if (dt == DT_F16) return f16_bits_to_f32(f32_to_f16_bits(x));
  return x;
}

DEV uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------- element access --

DEV const uint8_t* base_ptr(const KArgs& ka, uint32_t base) { return (const uint8_t*)ka.bases[base]; }

DEV float load_elem(const uint8_t* p, uint32_t dt, int64_t idx) {
  switch (dt) {
    case DT_F32: return ((const float*)p)[idx];
    case DT_BF16: return bf16_bits_to_f32(((const uint16_t*)p)[idx]);
    case DT_F16: return f16_bits_to_f32(((const uint16_t*)p)[idx]);
    default: return (float)((const int8_t*)p)[idx];
  }
}

DEV void store_elem(uint8_t* p, uint32_t dt, int64_t idx, float v) {
  switch (dt) {
    case DT_F32: ((float*)p)[idx] = v; break;
    case DT_BF16: ((uint16_t*)p)[idx] = (uint16_t)f32_to_bf16_bits(v); break;
    case DT_F16: ((uint16_t*)p)[idx] = (uint16_t)f32_to_f16_bits(v); break;
    default: break;
  }
}

// Element index of a view at coordinates c (dims past the task's rank have
// coordinate 0 and stride 0).
DEV int64_t view_index(const DView& v, const uint32_t (&c)[kMaxDims]) {
  int64_t idx = v.offset;
#pragma unroll
  for (int d = 0; d < kMaxDims; ++d) idx += (int64_t)c[d] * v.stride[d];
  return idx;
}

DEV int64_t inner_stride(const DView& v, uint32_t nd) {
  return nd <= 1 ? v.stride[0] : nd == 2 ? v.stride[1] : nd == 3 ? v.stride[2] : v.stride[3];
}

// Load W consecutive (along the innermost iteration dim) elements of a view.
template <int W>
DEV void load_view(const KArgs& ka, const DView& v, const uint32_t (&c)[kMaxDims], uint32_t nd, float (&x)[W]) {
  const uint8_t* p = base_ptr(ka, v.base);
  const int64_t idx = view_index(v, c);
  const int64_t s = inner_stride(v, nd);
  const uint32_t dt = v.dtype;
  if (W == 1) {
    x[0] = load_elem(p, dt, idx);
    return;
  }
  if (s == 0) {
    float a = load_elem(p, dt, idx);
#pragma unroll
    for (int j = 0; j < W; ++j) x[j] = a;
    return;
  }
  if (s == 1) {
    if (dt == DT_BF16 || dt == DT_F16) {
      const uint16_t* q = (const uint16_t*)p + idx;
      if (((uintptr_t)q & 15) == 0) {
        u32x4 r = *(const u32x4*)q;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = r[j] & 0xffffu, hi = r[j] >> 16;
          x[2 * j] = dt == DT_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
          x[2 * j + 1] = dt == DT_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
        }
        return;
      }
    } else if (dt == DT_F32) {
      const float* q = (const float*)p + idx;
      if (((uintptr_t)q & 15) == 0) {
        u32x4 r0 = *(const u32x4*)q;
        u32x4 r1 = *(const u32x4*)(q + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = __uint_as_float(r0[j]);
          x[4 + j] = __uint_as_float(r1[j]);
        }
        return;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < W; ++j) x[j] = load_elem(p, dt, idx + (int64_t)j * s);
}

template <int W>
DEV void store_view(const KArgs& ka, const DView& v, const uint32_t (&c)[kMaxDims], uint32_t nd, const float (&x)[W]) {
  uint8_t* p = (uint8_t*)ka.bases[v.base];
  const int64_t idx = view_index(v, c);
  const int64_t s = inner_stride(v, nd);
  const uint32_t dt = v.dtype;
  if (W == 8 && s == 1) {
    if (dt == DT_BF16 || dt == DT_F16) {
      uint16_t* q = (uint16_t*)p + idx;
      if (((uintptr_t)q & 15) == 0) {
        u32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t lo = dt == DT_BF16 ? f32_to_bf16_bits(x[2 * j]) : f32_to_f16_bits(x[2 * j]);
          uint32_t hi = dt == DT_BF16 ? f32_to_bf16_bits(x[2 * j + 1]) : f32_to_f16_bits(x[2 * j + 1]);
          r[j] = lo | (hi << 16);
        }
        *(u32x4*)q = r;
        return;
      }
    } else if (dt == DT_F32) {
      float* q = (float*)p + idx;
      if (((uintptr_t)q & 15) == 0) {
        u32x4 r0, r1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r0[j] = __float_as_uint(x[j]);
          r1[j] = __float_as_uint(x[4 + j]);
        }
        *(u32x4*)q = r0;
        *(u32x4*)(q + 4) = r1;
        return;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < W; ++j) store_elem(p, dt, idx + (int64_t)j * s, x[j]);
}

// ------------------------------------------------------ expression machine --

// The current stage's descriptors (in LDS when the stage blob fits).
struct Plan {
  const DTask* tasks;
  const DView* views;
  const DIns* ins;
};

template <int W>
struct Slots {
  float s0[W], s1[W], s2[W], s3[W];
  DEV void get(uint32_t k, float (&x)[W]) const {
    switch (k) {
      case 0:
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = s0[j];
        break;
      case 1:
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = s1[j];
        break;
      case 2:
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = s2[j];
        break;
      default:
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = s3[j];
        break;
    }
  }
  DEV void set(uint32_t k, const float (&x)[W]) {
    switch (k) {
      case 0:
#pragma unroll
        for (int j = 0; j < W; ++j) s0[j] = x[j];
        break;
      case 1:
#pragma unroll
        for (int j = 0; j < W; ++j) s1[j] = x[j];
        break;
      case 2:
#pragma unroll
        for (int j = 0; j < W; ++j) s2[j] = x[j];
        break;
      default:
#pragma unroll
        for (int j = 0; j < W; ++j) s3[j] = x[j];
        break;
    }
  }
};

// Run `n` instructions on the accumulator `acc` at chunk coordinates `c`.
template <int W>
DEV void vm_run(const KArgs& ka, const Plan& pl, uint32_t first, uint32_t n, const uint32_t (&c)[kMaxDims],
                uint32_t nd, float (&acc)[W]) {
  Slots<W> sl;
  for (uint32_t pc = 0; pc < n; ++pc) {
    const DIns in = pl.ins[first + pc];
    const uint32_t op = uniform(in.op), src = uniform(in.src), rnd = uniform(in.rnd), rev = uniform(in.rev);
    const uint32_t arg = uniform(in.arg);
    float x[W];
    if (src == SRC_VIEW) {
      load_view<W>(ka, pl.views[arg], c, nd, x);
    } else if (src == SRC_SCALAR) {
#pragma unroll
      for (int j = 0; j < W; ++j) x[j] = in.s;
    } else if (src == SRC_SLOT) {
      sl.get(arg, x);
    } else {
#pragma unroll
      for (int j = 0; j < W; ++j) x[j] = 0.0f;
    }
    const float a = in.a;
    switch (op) {
      case VM_LOAD:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = x[j];
        break;
      case VM_ADD:
#pragma unroll
        for (int j = 0; j < W; ++j) {
          if (rev) { float t = a * acc[j]; acc[j] = x[j] + t; }
          else { float t = a * x[j]; acc[j] = acc[j] + t; }
        }
        break;
      case VM_SUB:
#pragma unroll
        for (int j = 0; j < W; ++j) {
          if (rev) { float t = a * acc[j]; acc[j] = x[j] - t; }
          else { float t = a * x[j]; acc[j] = acc[j] - t; }
        }
        break;
      case VM_MUL:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = rev ? x[j] * acc[j] : acc[j] * x[j];
        break;
      case VM_DIV:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = rev ? x[j] / acc[j] : acc[j] / x[j];
        break;
      case VM_NEG:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = -acc[j];
        break;
      case VM_RELU:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = acc[j] < 0.0f ? 0.0f : acc[j];
        break;
      case VM_SQUARE:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = acc[j] * acc[j];
        break;
      case VM_POW:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = powf(acc[j], a);
        break;
      case VM_TB:
#pragma unroll
        for (int j = 0; j < W; ++j) {
          if (rev) acc[j] = acc[j] <= a ? 0.0f : x[j];
          else acc[j] = x[j] <= a ? 0.0f : acc[j];
        }
        break;
      case VM_SAVE:
        sl.set(arg, acc);
        break;
      case VM_STORE:
        store_view<W>(ka, pl.views[arg], c, nd, acc);
        break;
      case VM_SCALE:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = a * acc[j];
        break;
      case VM_ZERO:
#pragma unroll
        for (int j = 0; j < W; ++j) acc[j] = 0.0f;
        break;
      default:
        break;
    }
    if (rnd != RND_NONE) {
#pragma unroll
      for (int j = 0; j < W; ++j) acc[j] = round_to(acc[j], rnd);
    }
  }
}

DEV void unravel(uint32_t e, const DTask& t, uint32_t nd, uint32_t (&c)[kMaxDims]) {
#pragma unroll
  for (int d = kMaxDims - 1; d >= 0; --d) {
    if ((uint32_t)d >= nd) {
      c[d] = 0;
    } else {
      const uint32_t n = t.dims[d];
      c[d] = e % n;
      e /= n;
    }
  }
}

// ------------------------------------------------------------- elementwise --

template <int W>
__device__ __noinline__ void run_ew(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item) {
  const uint32_t nd = t.ndim;
  uint32_t numel = 1;
#pragma unroll
  for (int d = 0; d < kMaxDims; ++d) numel *= t.dims[d];  // unused dims are 1
  const uint32_t base = item * 2048u;
  if (W == 8) {
    const uint32_t e = base + threadIdx.x * 8u;
    if (e < numel) {
      uint32_t c[kMaxDims];
      unravel(e, t, nd, c);
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      vm_run<8>(ka, pl, t.expr_first, t.expr_len, c, nd, acc);
    }
  } else {
    for (uint32_t j = 0; j < 8; ++j) {
      const uint32_t e = base + j * 256u + threadIdx.x;
      if (e < numel) {
        uint32_t c[kMaxDims];
        unravel(e, t, nd, c);
        float acc[1] = {0};
        vm_run<1>(ka, pl, t.expr_first, t.expr_len, c, nd, acc);
      }
    }
  }
}

// Epilogue over a tile held in LDS as fp32 [BM][BN + 4].
template <int W>
DEV void tile_epilogue(const KArgs& ka, const Plan& pl, const DTask& t, const float* ctile, int BM, int BN,
                       uint32_t m0, uint32_t n0, uint32_t split_index) {
  const int pitch = BN + 4;
  const int cpr = BN / W;  // chunks per row
  const int nchunks = BM * cpr;
  const bool partial = (t.flags & F_PARTIAL) != 0;
  for (int q = threadIdx.x; q < nchunks; q += kBlock) {
    const int r = q / cpr, cc = (q % cpr) * W;
    const uint32_t row = m0 + r, col = n0 + cc;
    if (row >= t.m || col >= t.n) continue;
    float acc[W];
#pragma unroll
    for (int j = 0; j < W; ++j) acc[j] = ctile[r * pitch + cc + j];
    if (partial) {
      float* P = (float*)(ka.ws + t.scratch) + ((uint64_t)split_index * t.m + row) * t.n + col;
#pragma unroll
      for (int j = 0; j < W; ++j) P[j] = acc[j];
      continue;
    }
    uint32_t c[kMaxDims] = {row, col, 0, 0};
    vm_run<W>(ka, pl, t.expr_first, t.expr_len, c, 2, acc);
  }
}

// ------------------------------------------------------ fp32-FMA contraction --
// 64x64 output tile, 256 threads, each thread a 4x4 block; K staged 16 deep.
// Each output accumulates acc = fma(a_k, b_k, acc) for k = 0, 1, ... in order.

__device__ __noinline__ void run_gemm_simt(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  const uint32_t tm = item / t.tiles_n, tn = item % t.tiles_n;
  const uint32_t m0 = tm * 64, n0 = tn * 64;
  float* As = (float*)smem;              // [16][64 + 4]
  float* Bs = As + 16 * 68;              // [16][64 + 4]
  const DView A = pl.views[t.va], B = pl.views[t.vb];
  const uint8_t* pa = base_ptr(ka, A.base);
  const uint8_t* pb = base_ptr(ka, B.base);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (uint32_t k0 = 0; k0 < t.k; k0 += 16) {
    for (int p = threadIdx.x; p < 1024; p += kBlock) {
      const int kk = p % 16, mm = p / 16;  // A: 64 rows x 16 k
      const uint32_t gm = m0 + mm, gk = k0 + kk;
      As[kk * 68 + mm] = (gm < t.m && gk < t.k) ? load_elem(pa, A.dtype, A.offset + (int64_t)gm * A.stride[0] + (int64_t)gk * A.stride[1]) : 0.0f;
      const int nn = p % 64, kb = p / 64;  // B: 16 k x 64 cols
      const uint32_t gn = n0 + nn, gkb = k0 + kb;
      Bs[kb * 68 + nn] = (gn < t.n && gkb < t.k) ? load_elem(pb, B.dtype, B.offset + (int64_t)gkb * B.stride[0] + (int64_t)gn * B.stride[1]) : 0.0f;
    }
    __syncthreads();
    const uint32_t kend = t.k - k0 < 16 ? t.k - k0 : 16;
    for (uint32_t kk = 0; kk < kend; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk * 68 + ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk * 68 + tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = (float*)smem;  // [64][68]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) C[(ty * 4 + i) * 68 + tx * 4 + j] = acc[i][j];
  __syncthreads();
  if (t.width == 8)
    tile_epilogue<8>(ka, pl, t, C, 64, 64, m0, n0, 0);
  else
    tile_epilogue<1>(ka, pl, t, C, 64, 64, m0, n0, 0);
  __syncthreads();
}

// ------------------------------------------------------- MFMA contraction --
// Tile BM x BN, K staged 64 deep; 4 waves in a 2x2 grid, each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA accumulators.  Both operands are staged
// in LDS k-contiguous ([row][k], pitch 72 elements): an operand stored with
// unit stride along M/N is transposed in registers on its way to LDS so every
// global read stays 16 bytes wide and coalesced.

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;

// Stage rows [r0, r0 + R) x k [k0, k0 + 64) of an operand whose element (r, k)
// lives at p[off + r * sr + k * sk] into lds[r][k] (bf16/f16 bits).
template <int R>
DEV void stage_operand(const uint8_t* p, int64_t off, int64_t sr, int64_t sk, uint32_t r0, uint32_t rmax, uint32_t k0,
                       uint32_t kmax, uint16_t* lds) {
  const uint16_t* q = (const uint16_t*)p;
  if (sk == 1) {
    // 16-byte chunks along k: R * 8 chunks
#pragma unroll
    for (int i = 0; i < R / 32; ++i) {
      const int ch = threadIdx.x + i * kBlock;
      const int r = ch / 8, kq = (ch % 8) * 8;
      const uint32_t gr = r0 + r, gk = k0 + kq;
      const int64_t idx = off + (int64_t)gr * sr + gk;
      u32x4 v;
      if (gr < rmax && gk + 8 <= kmax && (((uintptr_t)(q + idx)) & 15) == 0) {
        v = *(const u32x4*)(q + idx);
      } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = (gr < rmax && gk + j < kmax) ? q[idx + j] : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = e[2 * j] | (e[2 * j + 1] << 16);
      }
      *(u32x4*)(lds + r * kPitch + kq) = v;
    }
  } else if (sr == 1) {
    // unit stride along rows: blocks of KB k-rows x 8 rows, transposed in registers
    constexpr int KB = R / 32;  // 4 for R = 128, 2 for R = 64
    const int rb = threadIdx.x % (R / 8), kb = threadIdx.x / (R / 8);
    const uint32_t gr = r0 + rb * 8, gk = k0 + kb * KB;
    uint32_t w[KB][4];
#pragma unroll
    for (int kr = 0; kr < KB; ++kr) {
      const int64_t idx = off + (int64_t)(gk + kr) * sk + gr;
      if (gk + kr < kmax && gr + 8 <= rmax && (((uintptr_t)(q + idx)) & 15) == 0) {
        u32x4 v = *(const u32x4*)(q + idx);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[kr][j] = v[j];
      } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = (gk + kr < kmax && gr + j < rmax) ? q[idx + j] : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[kr][j] = e[2 * j] | (e[2 * j + 1] << 16);
      }
    }
    // row rb*8 + 2j takes the low halves, row rb*8 + 2j + 1 the high halves
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo[KB / 2], hi[KB / 2];
#pragma unroll
      for (int h = 0; h < KB / 2; ++h) {
        lo[h] = (w[2 * h][j] & 0xffffu) | (w[2 * h + 1][j] << 16);
        hi[h] = (w[2 * h][j] >> 16) | (w[2 * h + 1][j] & 0xffff0000u);
      }
      uint16_t* d0 = lds + (rb * 8 + 2 * j) * kPitch + kb * KB;
      uint16_t* d1 = d0 + kPitch;
      if (KB == 4) {
        u32x2 a = {lo[0], lo[1]}, b = {hi[0], hi[1]};
        *(u32x2*)d0 = a;
        *(u32x2*)d1 = b;
      } else {
        *(uint32_t*)d0 = lo[0];
        *(uint32_t*)d1 = hi[0];
      }
    }
  } else {
    // general strides: element by element
    for (int p = threadIdx.x; p < R * kBK; p += kBlock) {
      const int r = p / kBK, kk = p % kBK;
      const uint32_t gr = r0 + r, gk = k0 + kk;
      lds[r * kPitch + kk] = (gr < rmax && gk < kmax) ? q[off + (int64_t)gr * sr + (int64_t)gk * sk] : (uint16_t)0;
    }
  }
}

template <bool BF16>
DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <bool BF16, int BM, int BN>
__device__ __noinline__ void run_gemm_mfma(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  constexpr int FM = BM / 64, FN = BN / 64;  // 32x32 blocks per wave along m / n
  const uint32_t tiles = t.tiles_m * t.tiles_n;
  const uint32_t split_index = item / tiles;
  const uint32_t tile = item % tiles;
  const uint32_t tm = tile / t.tiles_n, tn = tile % t.tiles_n;
  const uint32_t m0 = tm * BM, n0 = tn * BN;
  const uint32_t kbeg = split_index * t.kchunk;
  const uint32_t kend = (kbeg + t.kchunk < t.k) ? kbeg + t.kchunk : t.k;
  const DView A = pl.views[t.va], B = pl.views[t.vb];
  const uint8_t* pa = base_ptr(ka, A.base);
  const uint8_t* pb = base_ptr(ka, B.base);
  uint16_t* sa[2] = {(uint16_t*)smem, (uint16_t*)smem + BM * kPitch};
  uint16_t* sb[2] = {(uint16_t*)smem + 2 * BM * kPitch, (uint16_t*)smem + 2 * BM * kPitch + BN * kPitch};
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const uint32_t nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
  if (nk > 0) {
    stage_operand<BM>(pa, A.offset, A.stride[0], A.stride[1], m0, t.m, kbeg, kend, sa[0]);
    // B's element (n, k) lives at off + k * stride[0] + n * stride[1]
    stage_operand<BN>(pb, B.offset, B.stride[1], B.stride[0], n0, t.n, kbeg, kend, sb[0]);
  }
  __syncthreads();
  for (uint32_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      const uint32_t k1 = kbeg + (kt + 1) * kBK;
      stage_operand<BM>(pa, A.offset, A.stride[0], A.stride[1], m0, t.m, k1, kend, sa[cur ^ 1]);
      stage_operand<BN>(pb, B.offset, B.stride[1], B.stride[0], n0, t.n, k1, kend, sb[cur ^ 1]);
    }
    const uint16_t* a_t = sa[cur] + (wm * (BM / 2) + (lane % 32)) * kPitch + 8 * (lane / 32);
    const uint16_t* b_t = sb[cur] + (wn * (BN / 2) + (lane % 32)) * kPitch + 8 * (lane / 32);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const u32x4*)(a_t + i * 32 * kPitch + kk);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *(const u32x4*)(b_t + j * 32 * kPitch + kk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<BF16>(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }
  // accumulators -> LDS tile [BM][BN + 4]
  float* C = (float*)smem;
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
  __syncthreads();
  if (t.width == 8)
    tile_epilogue<8>(ka, pl, t, C, BM, BN, m0, n0, split_index);
  else
    tile_epilogue<1>(ka, pl, t, C, BM, BN, m0, n0, split_index);
  __syncthreads();
}

// Split-K combine: sum the partial tiles in split order, then the epilogue.
template <int W>
__device__ __noinline__ void run_gemm_reduce(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item) {
  const uint64_t total = (uint64_t)t.m * t.n;
  const float* P = (const float*)(ka.ws + t.scratch);
  for (uint32_t j8 = 0; j8 < (W == 8 ? 1u : 8u); ++j8) {
    const uint64_t e = (uint64_t)item * 2048u + (W == 8 ? threadIdx.x * 8u : j8 * 256u + threadIdx.x);
    if (e >= total) continue;
    const uint32_t row = (uint32_t)(e / t.n), col = (uint32_t)(e % t.n);
    float acc[W];
#pragma unroll
    for (int j = 0; j < W; ++j) acc[j] = P[e + j];
    for (uint32_t s = 1; s < t.split; ++s)
#pragma unroll
      for (int j = 0; j < W; ++j) acc[j] = acc[j] + P[s * total + e + j];
    uint32_t c[kMaxDims] = {row, col, 0, 0};
    vm_run<W>(ka, pl, t.expr_first, t.expr_len, c, 2, acc);
  }
}

// ------------------------------------------------------ int8-weight GEMV --
// 16 output rows per work item, 4 per wave; each lane takes 16-wide K chunks
// (k = 16 * lane + 1024 * j).  w = fl(q * s) then acc = fma(x, w, acc).

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __noinline__ void run_gemv_q8(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  const DView X = pl.views[t.va], Q = pl.views[t.vb], S = pl.views[t.vs];
  const uint8_t* px = base_ptr(ka, X.base);
  const int8_t* pq = (const int8_t*)base_ptr(ka, Q.base);
  const float* ps = (const float*)base_ptr(ka, S.base);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const uint32_t K = t.k;
  // The activation row, widened to fp32, staged once per item in LDS.
  float* xs = (float*)smem;
  const bool staged = (uint64_t)K * 4 + 64 <= (uint64_t)kSmemBytes;
  if (staged) {
    for (uint32_t k = threadIdx.x; k < K; k += kBlock)
      xs[k] = load_elem(px, X.dtype, X.offset + (int64_t)k * X.stride[1]);
    __syncthreads();
  }
  float* red = (float*)(smem + kSmemBytes - 64);
  for (int r = 0; r < 4; ++r) {
    const uint32_t row = item * 16 + wave * 4 + r;
    float acc = 0.0f;
    if (row < t.n) {
      const int64_t qrow = Q.offset + (int64_t)row * Q.stride[0];
      const int64_t srow = S.offset + (int64_t)row * S.stride[0];
      for (uint32_t kc = lane * 16; kc < K; kc += 1024) {
        // a 16-wide chunk starting at a multiple of 16 lies inside one 32-block
        const float sv = ps[srow + (int64_t)(kc / 32) * S.stride[1]];
        const int64_t qidx = qrow + (int64_t)kc * Q.stride[1];
        if (staged && Q.stride[1] == 1 && kc + 16 <= K && (((uintptr_t)(pq + qidx)) & 15) == 0) {
          const u32x4 v = *(const u32x4*)(pq + qidx);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int32_t qj = (int32_t)(v[j / 4] << (24 - 8 * (j % 4))) >> 24;
            const float w = (float)qj * sv;
            acc = __builtin_fmaf(xs[kc + j], w, acc);
          }
        } else {
          for (uint32_t j = 0; j < 16 && kc + j < K; ++j) {
            const float xj = staged ? xs[kc + j] : load_elem(px, X.dtype, X.offset + (int64_t)(kc + j) * X.stride[1]);
            const float w = (float)pq[qidx + (int64_t)j * Q.stride[1]] * sv;
            acc = __builtin_fmaf(xj, w, acc);
          }
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wave * 4 + r] = acc;
  }
  __syncthreads();
  const uint32_t rb = item * 16;
  if (t.width == 8) {
    if (threadIdx.x < 2) {
      const uint32_t col = rb + threadIdx.x * 8;
      if (col < t.n) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = red[threadIdx.x * 8 + j];
        uint32_t c[kMaxDims] = {0, col, 0, 0};
        vm_run<8>(ka, pl, t.expr_first, t.expr_len, c, 2, v);
      }
    }
  } else if (threadIdx.x < 16) {
    const uint32_t col = rb + threadIdx.x;
    if (col < t.n) {
      float v[1] = {red[threadIdx.x]};
      uint32_t c[kMaxDims] = {0, col, 0, 0};
      vm_run<1>(ka, pl, t.expr_first, t.expr_len, c, 2, v);
    }
  }
  __syncthreads();
}

// -------------------------------------------------------------- reductions --

// Block-wide sum in a fixed order: wave butterflies, then waves 0..3 in order.
DEV float block_sum(float v, float* scratch) {
  v = wave_sum(v);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float s = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
  __syncthreads();
  return s;
}

// Reduce the trailing part of the iteration space: item = row * parts + part.
template <int W>
__device__ __noinline__ void run_red_rows(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  const uint32_t row = item / t.split, part = item % t.split;
  const uint32_t R = t.k;
  const uint32_t kb = part * t.kchunk;
  const uint32_t ke = (kb + t.kchunk < R) ? kb + t.kchunk : R;
  const uint32_t nd = t.ndim;
  float s = 0.0f;
  for (uint32_t kk = kb + threadIdx.x * W; kk < ke; kk += kBlock * W) {
    const uint32_t e = row * R + kk;
    uint32_t c[kMaxDims];
    unravel(e, t, nd, c);
    float acc[W];
#pragma unroll
    for (int j = 0; j < W; ++j) acc[j] = 0.0f;
    vm_run<W>(ka, pl, t.expr_first, t.expr_len, c, nd, acc);
#pragma unroll
    for (int j = 0; j < W; ++j) s = s + acc[j];
  }
  const float total = block_sum(s, (float*)smem);
  if (threadIdx.x == 0) {
    if (t.flags & F_PARTIAL) {
      ((float*)(ka.ws + t.scratch))[(uint64_t)row * t.split + part] = total;
    } else {
      float v[1] = {total};
      uint32_t c[kMaxDims] = {row, 0, 0, 0};
      vm_run<1>(ka, pl, t.fin_first, t.fin_len, c, 1, v);
    }
  }
}

// Reduce the leading part: item = colblock * parts + part; 32 column chunks x
// 8 row lanes per workgroup, rows summed lane-strided then across lanes in order.
template <int W>
__device__ __noinline__ void run_red_cols(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  const uint32_t cb = item / t.split, part = item % t.split;
  const uint32_t cols = t.m, R = t.k;
  const uint32_t cc = threadIdx.x % 32, rl = threadIdx.x / 32;
  const uint32_t col = cb * 32 * W + cc * W;
  const uint32_t rb = part * t.kchunk;
  const uint32_t re = (rb + t.kchunk < R) ? rb + t.kchunk : R;
  const uint32_t nd = t.ndim;
  float s[W];
#pragma unroll
  for (int j = 0; j < W; ++j) s[j] = 0.0f;
  if (col < cols) {
    for (uint32_t r = rb + rl; r < re; r += 8) {
      const uint32_t e = r * cols + col;
      uint32_t c[kMaxDims];
      unravel(e, t, nd, c);
      float acc[W];
#pragma unroll
      for (int j = 0; j < W; ++j) acc[j] = 0.0f;
      vm_run<W>(ka, pl, t.expr_first, t.expr_len, c, nd, acc);
#pragma unroll
      for (int j = 0; j < W; ++j) s[j] = s[j] + acc[j];
    }
  }
  float* red = (float*)smem;  // [8][32 * W]
#pragma unroll
  for (int j = 0; j < W; ++j) red[rl * 32 * W + cc * W + j] = s[j];
  __syncthreads();
  if (rl == 0 && col < cols) {
    float tot[W];
#pragma unroll
    for (int j = 0; j < W; ++j) {
      float a = red[cc * W + j];
      for (int q = 1; q < 8; ++q) a = a + red[q * 32 * W + cc * W + j];
      tot[j] = a;
    }
    if (t.flags & F_PARTIAL) {
      float* P = (float*)(ka.ws + t.scratch) + (uint64_t)part * cols + col;
#pragma unroll
      for (int j = 0; j < W; ++j) P[j] = tot[j];
    } else {
      uint32_t c[kMaxDims] = {col, 0, 0, 0};
      vm_run<W>(ka, pl, t.fin_first, t.fin_len, c, 1, tot);
    }
  }
  __syncthreads();
}

__device__ __noinline__ void run_red_final(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item) {
  const uint32_t row = item * kBlock + threadIdx.x;
  if (row >= t.m) return;
  const float* P = (const float*)(ka.ws + t.scratch);
  float a = 0.0f;
  for (uint32_t p = 0; p < t.split; ++p) a = a + (t.tile ? P[(uint64_t)p * t.m + row] : P[(uint64_t)row * t.split + p]);
  float v[1] = {a};
  uint32_t c[kMaxDims] = {row, 0, 0, 0};
  vm_run<1>(ka, pl, t.fin_first, t.fin_len, c, 1, v);
}

// -------------------------------------------------------------- dispatch --

DEV void run_item(const KArgs& ka, const Plan& pl, const DTask& t, uint32_t item, uint8_t* smem) {
  switch (t.kind) {
    case T_EW:
      if (t.width == 8) run_ew<8>(ka, pl, t, item);
      else run_ew<1>(ka, pl, t, item);
      break;
    case T_GEMM_SIMT:
      run_gemm_simt(ka, pl, t, item, smem);
      break;
    case T_GEMM_MFMA: {
      const bool bf = pl.views[t.va].dtype == DT_BF16;
      if (t.tile == 0) {
        if (bf) run_gemm_mfma<true, 128, 128>(ka, pl, t, item, smem);
        else run_gemm_mfma<false, 128, 128>(ka, pl, t, item, smem);
      } else {
        if (bf) run_gemm_mfma<true, 64, 64>(ka, pl, t, item, smem);
        else run_gemm_mfma<false, 64, 64>(ka, pl, t, item, smem);
      }
      break;
    }
    case T_GEMM_REDUCE:
      if (t.width == 8) run_gemm_reduce<8>(ka, pl, t, item);
      else run_gemm_reduce<1>(ka, pl, t, item);
      break;
    case T_GEMV_Q8:
      run_gemv_q8(ka, pl, t, item, smem);
      break;
    case T_RED_ROWS:
      if (t.width == 8) run_red_rows<8>(ka, pl, t, item, smem);
      else run_red_rows<1>(ka, pl, t, item, smem);
      break;
    case T_RED_COLS:
      if (t.width == 8) run_red_cols<8>(ka, pl, t, item, smem);
      else run_red_cols<1>(ka, pl, t, item, smem);
      break;
    case T_RED_FINAL:
      run_red_final(ka, pl, t, item);
      break;
    default:
      break;
  }
}

// Grid barrier with per-workgroup flags.  Arrival: every wave waits for its
// own stores, the workgroup meets, one lane publishes (agent-scope release)
// and writes its arrival flag = epoch.  The first wave of workgroup 0 polls
// all arrival flags (4 per lane, loads issued together), then acquires and
// writes every workgroup's release flag; each other workgroup polls its own
// release flag and acquires.  No two workgroups spin on one address.  Epochs
// grow monotonically across launches on a workspace (the base is kept in the
// header), so flags never need resetting.  Every spin is bounded by the
// deadline; a timeout sets the abort word, which every spinner also watches.
DEV bool grid_barrier(const KArgs& ka, uint32_t epoch, uint32_t stage, uint64_t deadline) {
  __shared__ uint32_t s_ok;
  uint32_t* arrive = (uint32_t*)(ka.ws + kHdrArrive);
  uint32_t* release = (uint32_t*)(ka.ws + kHdrRelease);
  uint32_t* abort = (uint32_t*)(ka.ws + kHdrAbort);
  const uint32_t G = gridDim.x, bid = blockIdx.x;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(arrive + bid * kFlagStride, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (bid == 0 && threadIdx.x < 64) {
    uint32_t ok = 1;
    const uint32_t lane = threadIdx.x;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t base = 0; base < G; base += 256) {
      uint32_t* f[4];
      bool live[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = base + lane + 64 * i;
        live[i] = w < G;
        f[i] = arrive + (live[i] ? w : 0) * kFlagStride;
      }
      for (;;) {
        bool done = true;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (live[i]) {
            const uint32_t v = __hip_atomic_load(f[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((int32_t)(v - epoch) < 0) done = false;
          }
        if (done) break;
        if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = 0; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > deadline) {
          __hip_atomic_store((uint32_t*)(ka.ws + kHdrAbortStage), stage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
      }
      if (!ok) break;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
    // release everyone (a timed-out master still releases: the abort word stops them)
    for (uint32_t w = lane; w < G; w += 64)
      __hip_atomic_store(release + w * kFlagStride, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t all_ok = __builtin_amdgcn_readfirstlane(ok) & (uint32_t)__all(ok);
    if (lane == 0) s_ok = all_ok;
  } else if (bid != 0 && threadIdx.x == 0) {
    uint32_t ok = 1;
    uint32_t* f = release + bid * kFlagStride;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((int32_t)(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - epoch) < 0) {
      if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) { ok = 0; break; }
      if (__builtin_amdgcn_s_memrealtime() - t0 > deadline) {
        __hip_atomic_store((uint32_t*)(ka.ws + kHdrAbortStage), stage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok;
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

// Copy a stage blob into LDS (all threads; 16-byte chunks).
DEV void stage_blob_to_lds(const uint8_t* plan, const DStage& st, uint8_t* lds) {
  const u32x4* src = (const u32x4*)(plan + st.blob_off);
  u32x4* dst = (u32x4*)lds;
  for (uint32_t i = threadIdx.x; i < st.blob_bytes / 16; i += kBlock) dst[i] = src[i];
}

}  // namespace

__global__ __launch_bounds__(kBlock, 2) void tk_persistent(KArgs) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  __shared__ __attribute__((aligned(16))) uint8_t planbuf[kPlanLds];
  // Read the argument block in place (the kernarg segment) so the base-pointer
  // table is indexed in memory rather than copied into private storage.
  const KArgs& ka = *(const KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const DHeader* h = (const DHeader*)ka.plan;
  const DStage* stages = (const DStage*)(ka.plan + h->off_stages);
  const uint32_t n_stages = h->n_stages;
  const uint64_t deadline = ka.deadline_ticks ? ka.deadline_ticks : 400000000ull;  // 4 s at 100 MHz
  if (*(volatile uint32_t*)(ka.ws + kHdrAbort) != 0u) return;  // a previous launch on this workspace aborted
  const uint32_t epoch0 = *(volatile uint32_t*)(ka.ws + kHdrEpoch);
  if (n_stages == 0) return;
  DStage st = stages[0];
  if (st.blob_bytes <= kPlanLds) stage_blob_to_lds(ka.plan, st, planbuf);
  __syncthreads();
  for (uint32_t s = 0; s < n_stages; ++s) {
    const bool in_lds = st.blob_bytes <= kPlanLds;
    const uint8_t* blob = in_lds ? planbuf : ka.plan + st.blob_off;
    Plan pl;
    pl.tasks = (const DTask*)blob;
    pl.views = (const DView*)(blob + st.off_views);
    pl.ins = (const DIns*)(blob + st.off_ins);
    uint32_t ti = 0;
    for (uint32_t item = blockIdx.x; item < st.n_items; item += gridDim.x) {
      while (ti + 1 < st.n_tasks && item >= pl.tasks[ti + 1].item_begin) ++ti;
      const DTask t = pl.tasks[ti];
      if (ka.flags & K_STAGGER) {
        uint32_t n = hash32(ka.stagger_seed ^ (blockIdx.x * 0x9e3779b9u) ^ (item * 0x85ebca6bu) ^ s) % 48u;
        for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
      }
      run_item(ka, pl, t, item - t.item_begin, smem);
    }
    if (s + 1 < n_stages) {
      // stage the next stage's descriptors while the barrier completes
      __syncthreads();
      st = stages[s + 1];
      if (st.blob_bytes <= kPlanLds) stage_blob_to_lds(ka.plan, st, planbuf);
      const bool stamp = (ka.flags & K_TIMESTAMPS) && blockIdx.x == 0 && threadIdx.x == 0 && s < kMaxTimedStages;
      if (stamp) ((uint64_t*)(ka.ws + kHdrStamps))[2 * s] = __builtin_amdgcn_s_memrealtime();
      if (!grid_barrier(ka, epoch0 + s + 1, s, deadline)) return;
      if (stamp) ((uint64_t*)(ka.ws + kHdrStamps))[2 * s + 1] = __builtin_amdgcn_s_memrealtime();
    }
  }
  // The next launch on this workspace continues the epoch sequence.  Every
  // workgroup has read the base before the first barrier, which this
  // workgroup has passed.
  if (n_stages > 1 && blockIdx.x == 0 && threadIdx.x == 0)
    *(volatile uint32_t*)(ka.ws + kHdrEpoch) = epoch0 + n_stages - 1;
}

__global__ void tk_zero_header(uint8_t* ws, uint32_t bytes) {
  for (uint32_t i = threadIdx.x * 4; i < bytes; i += blockDim.x * 4) *(uint32_t*)(ws + i) = 0u;
}

// Host-side launch helpers used by the C ABI.
hipError_t tk_device_launch(const KArgs& ka, int grid, hipStream_t stream) {
  void* args[] = {(void*)&ka};
  return hipLaunchCooperativeKernel((const void*)tk_persistent, dim3(grid), dim3(kBlock), args, 0, stream);
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
