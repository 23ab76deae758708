// tk_oracle -- TEST INFRASTRUCTURE ONLY.  The plain CPU reference for the
// whole-step programs.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg may load it; the product library never does.  It shares no
// code with the HIP library: its own parser, its own rounding, its own loops.
//
// What it computes (trainkernel pages: codegen.py, the module docstring and
// `_Generator.generate`): the program's operations run one after another in
// their listed (topological) order; every operation's value is rounded to its
// output dtype (`_round` / `store`); returned values are converted to their
// output spec's dtype through their view (output-copy stage of `generate`);
// in-place outputs are written into their input's memory only after every
// operation has run (the transactional commit at the end of `generate`).
//
// Arithmetic is IEEE-754 binary32 with round-to-nearest-even and no fused
// multiply-add except where a definition names one: the contractions
// accumulate `acc = fma(a, b, acc)` sequentially over k from +0 (the direct and
// SIMT matrix paths of `emit_mm`), and the page compiles with --fmad=false
// (runtime.py, `compile_program`).  Build with -ffp-contract=off, no fast-math.
//
// Mode 1 ("binary64") evaluates every value in double precision with no
// rounding to storage dtypes; all caller buffers are then arrays of double.
// It exists for the finite-difference checks of the explicit backward graphs.
//
// Parity pins (tests/test_oracle_*.py): exhaustive float->bf16/f16 rounding
// against library conversions, IEEE special cases of every pointwise op, exact
// integer matmuls and Higham's bound, exact reductions, finite differences and
// a hand-derived gradient of tiny MLPs, SGD closed forms, and invariants.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <sstream>
#include <stdexcept>
#include <string>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum DType { F32, F16, BF16, I8 };

struct View {
  std::string buf;
  DType dtype = F32;
  std::vector<int64_t> shape, strides;
  int64_t offset = 0;
};

struct Operand {
  bool is_scalar = false;
  float scalar = 0.0f;
  View view;
};

struct Op {
  std::string name, opcode;
  View out;
  std::vector<Operand> args;
  std::map<std::string, float> attrs;
  bool dims_all = true;
  std::vector<int64_t> dims;
};

struct Prog {
  std::vector<View> inputs;
  std::vector<Op> ops;
  std::vector<View> outputs;
  std::map<int, int> inplace;
};

[[noreturn]] void fail(const std::string& msg) { throw std::runtime_error("tk oracle: " + msg); }

int64_t numel(const std::vector<int64_t>& s) {
  int64_t n = 1;
  for (auto d : s) n *= d;
  return n;
}

// ----------------------------------------------------------------- parsing --

DType parse_dtype(const std::string& s) {
  if (s == "f32") return F32;
  if (s == "f16") return F16;
  if (s == "bf16") return BF16;
  if (s == "i8") return I8;
  fail("unsupported dtype " + s);
}

std::vector<int64_t> parse_dims(const std::string& s) {
  std::vector<int64_t> out;
  if (s == "-") return out;
  size_t pos = 0;
  while (pos <= s.size()) {
    size_t next = s.find('x', pos);
    std::string part = s.substr(pos, next == std::string::npos ? std::string::npos : next - pos);
    if (part.empty()) fail("bad dims '" + s + "'");
    char* end = nullptr;
    long long v = std::strtoll(part.c_str(), &end, 10);
    if (*end) fail("bad dims '" + s + "'");
    out.push_back(v);
    if (next == std::string::npos) break;
    pos = next + 1;
  }
  return out;
}

float parse_scalar(const std::string& s) {
  if (s.empty() || s[0] != '#') fail("bad scalar '" + s + "'");
  char* end = nullptr;
  double v = std::strtod(s.c_str() + 1, &end);  // hex floats are exact
  if (*end) fail("bad scalar '" + s + "'");
  float f = (float)v;
  if ((double)f != v) fail("scalar is not a float32 value: " + s);
  if (!std::isfinite(f)) fail("non-finite scalar constants are unsupported");
  return f;
}

View parse_spec(const std::string& s) {
  std::vector<std::string> f;
  size_t pos = 0;
  for (;;) {
    size_t n = s.find(':', pos);
    f.push_back(s.substr(pos, n == std::string::npos ? std::string::npos : n - pos));
    if (n == std::string::npos) break;
    pos = n + 1;
  }
  if (f.size() != 5) fail("bad spec '" + s + "'");
  View v;
  v.buf = f[0];
  v.dtype = parse_dtype(f[1]);
  v.shape = parse_dims(f[2]);
  v.strides = parse_dims(f[3]);
  v.offset = std::strtoll(f[4].c_str(), nullptr, 10);
  if (v.shape.size() != v.strides.size()) fail("rank of shape and strides differ in '" + s + "'");
  for (auto d : v.shape)
    if (d < 0) fail("negative dimension");
  for (auto d : v.strides)
    if (d < 0) fail("negative stride");
  if (v.offset < 0) fail("negative offset");
  return v;
}

Prog parse(const std::string& text) {
  Prog p;
  std::istringstream in(text);
  std::string line;
  bool header = false, ended = false;
  while (std::getline(in, line)) {
    auto c = line.find(';');
    if (c != std::string::npos) line = line.substr(0, c);
    std::istringstream ls(line);
    std::vector<std::string> tok;
    std::string t;
    while (ls >> t) tok.push_back(t);
    if (tok.empty()) continue;
    if (!header) {
      if (tok.size() != 2 || tok[0] != "tkir" || tok[1] != "1") fail("missing 'tkir 1' header");
      header = true;
      continue;
    }
    if (ended) fail("text after 'end'");
    if (tok[0] == "in") {
      if (tok.size() != 6) fail("bad input line");
      View v;
      v.buf = tok[1];
      v.dtype = parse_dtype(tok[2]);
      v.shape = parse_dims(tok[3]);
      v.strides = parse_dims(tok[4]);
      v.offset = std::strtoll(tok[5].c_str(), nullptr, 10);
      if (v.shape.size() != v.strides.size()) fail("input rank mismatch");
      p.inputs.push_back(v);
    } else if (tok[0] == "op") {
      if (tok.size() < 4) fail("bad op line");
      Op op;
      op.name = tok[1];
      op.opcode = tok[2];
      op.out = parse_spec(tok[3]);
      for (size_t i = 4; i < tok.size(); ++i) {
        const std::string& a = tok[i];
        auto eq = a.find('=');
        if (eq != std::string::npos) {
          std::string key = a.substr(0, eq), val = a.substr(eq + 1);
          if (key == "dims") {
            if (val == "all") {
              op.dims_all = true;
            } else {
              op.dims_all = false;
              size_t q = 0;
              while (q < val.size()) {
                size_t n = val.find(',', q);
                op.dims.push_back(std::strtoll(val.substr(q, n - q).c_str(), nullptr, 10));
                if (n == std::string::npos) break;
                q = n + 1;
              }
            }
          } else {
            op.attrs[key] = parse_scalar(val);
          }
        } else if (a[0] == '#') {
          Operand o;
          o.is_scalar = true;
          o.scalar = parse_scalar(a);
          op.args.push_back(o);
        } else {
          Operand o;
          o.view = parse_spec(a);
          op.args.push_back(o);
        }
      }
      p.ops.push_back(op);
    } else if (tok[0] == "out") {
      if (tok.size() != 2) fail("bad out line");
      p.outputs.push_back(parse_spec(tok[1]));
    } else if (tok[0] == "inplace") {
      if (tok.size() != 3) fail("bad inplace line");
      p.inplace[std::atoi(tok[1].c_str())] = std::atoi(tok[2].c_str());
    } else if (tok[0] == "end") {
      ended = true;
    } else {
      fail("unknown statement " + tok[0]);
    }
  }
  if (!header || !ended) fail("incomplete program text");
  return p;
}

// ---------------------------------------------------------------- rounding --
// Round-to-nearest-even from a float32 to a narrower IEEE-style format with
// `mbits` stored mantissa bits and exponent bias `bias` (max biased exponent
// 2*bias+1 reserved for Inf/NaN).  Written from the IEEE-754 definition of
// roundTiesToEven: scale the exact value to the target's unit in the last
// place, round the integer significand, renormalise, saturate to Inf.

uint16_t round_narrow(float x, int mbits, int ebits) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 31) & 1u;
  const int exp = (int)((u >> 23) & 0xffu);
  const uint32_t mant = u & 0x7fffffu;
  const int bias = (1 << (ebits - 1)) - 1;
  const uint32_t emax_field = (1u << ebits) - 1u;
  const uint32_t sign_out = sign << (mbits + ebits);
  if (exp == 0xff) {
    if (mant == 0) return (uint16_t)(sign_out | (emax_field << mbits));
    // NaN: keep it a quiet NaN, keeping the top payload bits.
    return (uint16_t)(sign_out | (emax_field << mbits) | (1u << (mbits - 1)) | (mant >> (23 - mbits)));
  }
  if (exp == 0 && mant == 0) return (uint16_t)sign_out;
  // value = sig * 2^(e2), sig a 24-bit integer (implicit bit made explicit)
  uint64_t sig = exp ? ((1u << 23) | mant) : mant;
  int e2 = exp ? exp - 127 - 23 : -126 - 23;
  // Normalise so the leading one is at bit 23.
  while (sig < (1u << 23)) {
    sig <<= 1;
    e2 -= 1;
  }
  int unbiased = e2 + 23;          // exponent of the leading one
  int target_e = unbiased + bias;  // biased target exponent if normal
  int drop;                        // number of low bits of `sig` to discard
  if (target_e >= 1) {
    drop = 23 - mbits;
  } else {
    drop = 23 - mbits + (1 - target_e);  // subnormal: fixed unit 2^(1-bias-mbits)
    target_e = 0;
  }
  uint64_t q;
  if (drop >= 64) {
    q = 0;
  } else if (drop > 25) {
    q = 0;  // below half of the smallest subnormal
  } else {
    q = sig >> drop;
    uint64_t rem = sig & ((1ull << drop) - 1);
    uint64_t half = 1ull << (drop - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
  }
  // q is the significand in units of the target ulp.  For normals it has
  // mbits+1 bits; a carry out moves to the next binade.
  uint32_t field;
  if (target_e >= 1) {
    if (q >> (mbits + 1)) {
      q >>= 1;
      target_e += 1;
    }
    if (target_e >= (int)emax_field) return (uint16_t)(sign_out | (emax_field << mbits));
    field = ((uint32_t)target_e << mbits) | (uint32_t)(q & ((1u << mbits) - 1));
  } else {
    field = (uint32_t)q;  // q == 2^mbits encodes the smallest normal exactly
  }
  return (uint16_t)(sign_out | field);
}

float widen_narrow(uint16_t h, int mbits, int ebits) {
  const uint32_t sign = (h >> (mbits + ebits)) & 1u;
  const uint32_t e = (h >> mbits) & ((1u << ebits) - 1u);
  const uint32_t m = h & ((1u << mbits) - 1u);
  const int bias = (1 << (ebits - 1)) - 1;
  double v;
  if (e == (1u << ebits) - 1u) {
    v = m ? NAN : INFINITY;
  } else if (e == 0) {
    v = std::ldexp((double)m, 1 - bias - mbits);
  } else {
    v = std::ldexp((double)((1u << mbits) | m), (int)e - bias - mbits);
  }
  return (float)(sign ? -v : v);
}

uint16_t to_bf16(float x) { return round_narrow(x, 7, 8); }
uint16_t to_f16(float x) { return round_narrow(x, 10, 5); }
float from_bf16(uint16_t h) { return widen_narrow(h, 7, 8); }
float from_f16(uint16_t h) { return widen_narrow(h, 10, 5); }

float round_to(DType t, float x) {
  switch (t) {
    case F32: return x;
    case BF16: return from_bf16(to_bf16(x));
    case F16: return from_f16(to_f16(x));
    default: fail("values cannot be rounded to int8");
  }
}

// ------------------------------------------------------------- evaluation --

template <class T>
struct Value {
  // Either a program input (raw caller memory of `dtype`, or double in mode 1)
  // or a computed op result (contiguous T array).
  const void* raw = nullptr;
  DType dtype = F32;
  std::vector<T> data;
  std::vector<int64_t> shape;
  bool computed = false;
};

template <class T>
struct Interp {
  const Prog& p;
  bool wide;  // binary64 mode
  std::map<std::string, Value<T>> vals;

  Interp(const Prog& prog, bool wide_mode) : p(prog), wide(wide_mode) {}

  T load_raw(const Value<T>& v, int64_t idx) const {
    if (v.computed) return v.data[idx];
    if (wide) return (T)static_cast<const double*>(v.raw)[idx];
    switch (v.dtype) {
      case F32: return (T) static_cast<const float*>(v.raw)[idx];
      case BF16: return (T)from_bf16(static_cast<const uint16_t*>(v.raw)[idx]);
      case F16: return (T)from_f16(static_cast<const uint16_t*>(v.raw)[idx]);
      case I8: return (T) static_cast<const int8_t*>(v.raw)[idx];
    }
    return 0;
  }

  const Value<T>& value_of(const View& v) const {
    auto it = vals.find(v.buf);
    if (it == vals.end()) fail("operand '" + v.buf + "' is not defined before use");
    return it->second;
  }

  // Extent check: every element the view can address must lie in its buffer.
  void check_view(const View& v) const {
    const Value<T>& src = value_of(v);
    if (numel(v.shape) == 0) return;
    int64_t hi = v.offset;
    for (size_t i = 0; i < v.shape.size(); ++i) hi += (v.shape[i] - 1) * v.strides[i];
    if (src.computed) {
      if (hi >= (int64_t)src.data.size()) fail("view of '" + v.buf + "' exceeds its extent");
    }
  }

  // Read operand view `v` at output coordinate `coord` (output rank R): the
  // view's dims align to the trailing output dims; size-1 dims broadcast.
  T read(const View& v, const std::vector<int64_t>& coord) const {
    const Value<T>& src = value_of(v);
    const size_t R = coord.size(), r = v.shape.size();
    int64_t idx = v.offset;
    for (size_t i = 0; i < r; ++i) {
      int64_t c = coord[R - r + i];
      if (v.shape[i] == 1) c = 0;
      idx += c * v.strides[i];
    }
    return load_raw(src, idx);
  }

  // Element (i, j) of a rank-two view whose buffer `src` was looked up once.
  T read2(const Value<T>& src, const View& v, int64_t i, int64_t j) const {
    return load_raw(src, v.offset + i * v.strides[0] + j * v.strides[1]);
  }

  void check_broadcast(const View& v, const std::vector<int64_t>& out) const {
    if (v.shape.size() > out.size()) fail("invalid broadcast rank");
    const size_t off = out.size() - v.shape.size();
    for (size_t i = 0; i < v.shape.size(); ++i)
      if (v.shape[i] != 1 && v.shape[i] != out[off + i]) fail("incompatible broadcast dimensions");
    check_view(v);
  }

  T rnd(DType t, T x) const {
    if (wide) return x;
    return (T)round_to(t, (float)x);
  }

  static void unravel(int64_t i, const std::vector<int64_t>& shape, std::vector<int64_t>& c) {
    c.resize(shape.size());
    for (size_t d = shape.size(); d-- > 0;) {
      int64_t n = shape[d] > 0 ? shape[d] : 1;
      c[d] = i % n;
      i /= n;
    }
  }

  T pointwise(const Op& op, const std::vector<int64_t>& coord) const {
    auto arg = [&](size_t i) -> T {
      const Operand& o = op.args.at(i);
      return o.is_scalar ? (T)o.scalar : read(o.view, coord);
    };
    auto attr = [&](const char* k, float dflt) -> T {
      auto it = op.attrs.find(k);
      return (T)(it == op.attrs.end() ? dflt : it->second);
    };
    const std::string& c = op.opcode;
    if (c == "add") { T b = attr("alpha", 1.0f) * arg(1); return arg(0) + b; }
    if (c == "sub") { T b = attr("alpha", 1.0f) * arg(1); return arg(0) - b; }
    if (c == "mul") return arg(0) * arg(1);
    if (c == "div") return arg(0) / arg(1);
    if (c == "neg") return -arg(0);
    if (c == "relu") { T x = arg(0); return x < (T)0 ? (T)0 : x; }
    if (c == "sqrt") return std::sqrt(arg(0));  // IEEE: correctly rounded in the evaluation type
    if (c == "pow") {
      T e = op.args.size() > 1 ? arg(1) : attr("exponent", 2.0f);
      T x = arg(0);
      if (e == (T)2) return x * x;
      return (T)std::pow(x, e);
    }
    if (c == "threshold_backward") {
      T g = arg(0), x = arg(1);
      return x <= attr("threshold", 0.0f) ? (T)0 : g;
    }
    if (c == "full") {
      // The `value` attribute wins; otherwise a scalar first operand; else 0.
      if (op.attrs.count("value")) return (T)op.attrs.at("value");
      if (!op.args.empty()) {
        if (!op.args[0].is_scalar) fail("full takes a scalar value");
        return (T)op.args[0].scalar;
      }
      return (T)0;
    }
    if (c == "cast") return arg(0);
    fail("unsupported pointwise operation " + c);
  }

  void run_pointwise(const Op& op, Value<T>& out) {
    static const char* known[] = {"add", "sub", "mul", "div", "neg", "relu", "pow", "threshold_backward", "full", "cast",
                                  "sqrt"};
    bool ok = false;
    for (const char* k : known) ok = ok || op.opcode == k;
    if (!ok) fail("unsupported pointwise operation " + op.opcode);
    static const char* unary[] = {"neg", "relu", "cast", "sqrt"};
    for (const char* k : unary)
      if (op.opcode == k && op.args.size() != 1) fail(op.opcode + " takes one operand");
    if ((op.opcode == "add" || op.opcode == "sub" || op.opcode == "mul" || op.opcode == "div" ||
         op.opcode == "threshold_backward") && op.args.size() != 2)
      fail(op.opcode + " takes two operands");
    for (auto& a : op.args)
      if (!a.is_scalar) check_broadcast(a.view, op.out.shape);
    if (op.opcode == "pow" && op.args.size() > 1 && !op.args[1].is_scalar) fail("pow exponent must be a scalar");
    const int64_t n = numel(op.out.shape);
    out.data.assign(n, 0);
#pragma omp parallel
    {
      std::vector<int64_t> coord;
#pragma omp for schedule(static)
      for (int64_t i = 0; i < n; ++i) {
        unravel(i, op.out.shape, coord);
        out.data[i] = rnd(op.out.dtype, pointwise(op, coord));
      }
    }
  }

  static T fma_(T a, T b, T c) { return std::fma(a, b, c); }

  // Q8_0 quantisation of activation row r (blocks of 32 along k, the last one
  // possibly shorter): d = amax / 127 in the working precision, each code the
  // quotient x / d rounded to the nearest integer (ties to even) and held in
  // [-127, 127]; an all-zero block has d = 0 and codes 0.  Finite inputs.
  void quantise_row(const Value<T>& VA, const View& A, int64_t r, int64_t k, std::vector<int32_t>& code,
                    std::vector<T>& scale) {
    const int64_t nb = (k + 31) / 32;
    code.assign(k, 0);
    scale.assign(nb, 0);
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t k0 = b * 32, k1 = std::min<int64_t>(k, k0 + 32);
      T amax = 0;
      for (int64_t kk = k0; kk < k1; ++kk) {
        const T a = std::fabs(read2(VA, A, r, kk));
        if (a > amax) amax = a;
      }
      const T d = amax / (T)127;
      scale[b] = d;
      if (d == (T)0) continue;
      for (int64_t kk = k0; kk < k1; ++kk) {
        const T q = std::nearbyint(read2(VA, A, r, kk) / d);
        code[kk] = (int32_t)std::max((T)-127, std::min((T)127, q));
      }
    }
  }

  void run_mm(const Op& op, Value<T>& out) {
    const bool add = op.opcode == "addmm" || op.opcode == "addmm_q8";
    const bool q8 = op.opcode == "mm_q8" || op.opcode == "addmm_q8";
    const size_t first = add ? 1 : 0;
    if (op.args.size() != first + (q8 ? 3 : 2)) fail("wrong operand count for " + op.opcode);
    for (size_t i = 0; i < op.args.size(); ++i)
      if (op.args[i].is_scalar) fail("matrix operands must be tensors");
    const View& A = op.args[first].view;
    const View& B = op.args[first + 1].view;
    if (A.shape.size() != 2 || B.shape.size() != 2) fail("mm requires rank-two tensors");
    check_view(A);
    check_view(B);
    const int64_t m = A.shape[0], k = A.shape[1];
    int64_t n;
    const View* S = nullptr;
    if (q8) {
      // B is the int8 weight [n, k]; S the float scales [n, ceil(k/32)].
      S = &op.args[first + 2].view;
      n = B.shape[0];
      if (B.shape[1] != k || B.dtype != I8) fail("q8 weight must be int8 [n, k]");
      if (S->shape.size() != 2 || S->shape[0] != n || S->shape[1] != (k + 31) / 32) fail("q8 scales must be [n, ceil(k/32)]");
      check_view(*S);
    } else {
      if (B.shape[0] != k) fail("mm requires compatible rank-two tensors");
      n = B.shape[1];
    }
    if (op.out.shape.size() != 2 || op.out.shape[0] != m || op.out.shape[1] != n)
      fail("matrix output shape does not match its inputs");
    const T alpha = (T)(op.attrs.count("alpha") ? op.attrs.at("alpha") : 1.0f);
    const T beta = (T)(op.attrs.count("beta") ? op.attrs.at("beta") : 1.0f);
    // xq: the activation rows are themselves quantised to Q8_0 before the
    // product (the decode lane's activation quantisation step, `lk_quant`, in
    // the emit.rs page's launch list).
    const bool xq = q8 && op.attrs.count("xq") && op.attrs.at("xq") != 0.0f;
    if (op.attrs.count("xq") && !q8) fail("xq applies to the q8 products only");
    const View* bias = add ? &op.args[0].view : nullptr;
    if (bias) check_broadcast(*bias, op.out.shape);
    out.data.assign(m * n, 0);
    const Value<T>& VA = value_of(A);
    const Value<T>& VB = value_of(B);
    const Value<T>* VS = q8 ? &value_of(*S) : nullptr;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r) {
      std::vector<int64_t> coord(2);
      std::vector<int32_t> xcode;
      std::vector<T> xscale;
      if (xq) quantise_row(VA, A, r, k, xcode, xscale);
      for (int64_t c = 0; c < n; ++c) {
        T acc = 0;
        if (xq) {
          // Q8_0 x Q8_0: per 32-block an exact integer dot product of the
          // codes, weighted by the product of the two block scales
          for (int64_t b = 0; b * 32 < k; ++b) {
            int64_t idot = 0;
            for (int64_t kk = b * 32; kk < k && kk < b * 32 + 32; ++kk)
              idot += (int64_t)xcode[kk] * (int64_t)read2(VB, B, c, kk);
            const T w = xscale[b] * read2(*VS, *S, c, b);
            acc = fma_(w, (T)idot, acc);
          }
        }
        for (int64_t kk = 0; kk < (xq ? 0 : k); ++kk) {
          T a = read2(VA, A, r, kk);
          T b;
          if (q8) {
            T qv = read2(VB, B, c, kk);
            T sv = read2(*VS, *S, c, kk / 32);
            b = qv * sv;  // dequantised weight, rounded to the working precision
          } else {
            b = read2(VB, B, kk, c);
          }
          acc = fma_(a, b, acc);
        }
        T v;
        if (!add) {
          v = acc;
        } else {
          coord[0] = r;
          coord[1] = c;
          if (alpha == (T)0 && beta == (T)0) {
            v = 0;
          } else if (beta == (T)0) {
            v = alpha * acc;
          } else if (alpha == (T)0) {
            v = beta * read(*bias, coord);
          } else {
            T s = alpha * acc;
            T t = beta * read(*bias, coord);
            v = s + t;
          }
        }
        out.data[r * n + c] = rnd(op.out.dtype, v);
      }
    }
  }

  void run_reduce(const Op& op, Value<T>& out) {
    if (op.args.size() != 1 || op.args[0].is_scalar) fail("reduction requires a tensor");
    const View& X = op.args[0].view;
    check_view(X);
    const int64_t rank = (int64_t)X.shape.size();
    std::vector<int64_t> dims;
    if (op.dims_all) {
      for (int64_t d = 0; d < rank; ++d) dims.push_back(d);
    } else {
      for (int64_t d : op.dims) {
        if (rank == 0) fail("cannot reduce a rank-zero tensor over explicit dims");
        dims.push_back(((d % rank) + rank) % rank);
      }
    }
    std::vector<bool> red(rank, false);
    for (auto d : dims) red[d] = true;
    std::vector<int64_t> kept_shape, red_shape, kept_idx, red_idx;
    for (int64_t d = 0; d < rank; ++d) {
      if (red[d]) {
        red_shape.push_back(X.shape[d]);
        red_idx.push_back(d);
      } else {
        kept_shape.push_back(X.shape[d]);
        kept_idx.push_back(d);
      }
    }
    if (numel(op.out.shape) != numel(kept_shape)) fail("reduction output shape does not match its axes");
    const int64_t rows = numel(kept_shape), size = numel(red_shape);
    const bool mean = op.opcode == "mean";
    out.data.assign(rows, 0);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
      std::vector<int64_t> kc, rc, coord(rank);
      unravel(row, kept_shape, kc);
      T acc = 0;
      for (int64_t r = 0; r < size; ++r) {
        unravel(r, red_shape, rc);
        for (size_t i = 0; i < kept_idx.size(); ++i) coord[kept_idx[i]] = kc[i];
        for (size_t i = 0; i < red_idx.size(); ++i) coord[red_idx[i]] = rc[i];
        acc = acc + read(X, coord);
      }
      T v = mean ? acc / (T)size : acc;  // empty mean is 0/0 = NaN
      out.data[row] = rnd(op.out.dtype, v);
    }
  }

  static bool contiguous(const View& v) {
    int64_t acc = 1;
    for (size_t d = v.shape.size(); d-- > 0;) {
      if (v.shape[d] != 1 && v.strides[d] != acc) return false;
      acc *= v.shape[d];
    }
    return true;
  }

  void run(const void* const* inputs, void* const* outputs) {
    for (size_t i = 0; i < p.inputs.size(); ++i) {
      const View& s = p.inputs[i];
      if (vals.count(s.buf)) fail("duplicate buffer name " + s.buf);
      Value<T> v;
      v.raw = inputs[i];
      v.dtype = s.dtype;
      v.shape = s.shape;
      vals[s.buf] = std::move(v);
    }
    for (const Op& op : p.ops) {
      if (vals.count(op.out.buf)) fail("buffer '" + op.out.buf + "' is defined twice");
      if (op.out.dtype == I8) fail("operations produce float values only");
      if (!contiguous(op.out) || op.out.offset != 0) fail("operation output must be contiguous: " + op.name);
      Value<T> v;
      v.computed = true;
      v.dtype = op.out.dtype;
      v.shape = op.out.shape;
      const std::string& c = op.opcode;
      if (c == "mm" || c == "addmm" || c == "mm_q8" || c == "addmm_q8")
        run_mm(op, v);
      else if (c == "sum" || c == "mean")
        run_reduce(op, v);
      else
        run_pointwise(op, v);
      vals[op.out.buf] = std::move(v);
    }
    // Gather every returned value first, then write: in-place outputs land in
    // their input's memory only after all reads (transactional commit).
    std::vector<std::vector<T>> results(p.outputs.size());
    for (size_t o = 0; o < p.outputs.size(); ++o) {
      const View& s = p.outputs[o];
      check_view(s);
      const int64_t n = numel(s.shape);
      results[o].resize(n);
      std::vector<int64_t> coord;
      for (int64_t i = 0; i < n; ++i) {
        unravel(i, s.shape, coord);
        int64_t idx = s.offset;
        for (size_t d = 0; d < s.shape.size(); ++d) idx += coord[d] * s.strides[d];
        results[o][i] = load_raw(value_of(s), idx);
      }
    }
    for (size_t o = 0; o < p.outputs.size(); ++o) {
      const View& s = p.outputs[o];
      const int64_t n = (int64_t)results[o].size();
      if (wide) {
        double* dst = static_cast<double*>(outputs[o]);
        for (int64_t i = 0; i < n; ++i) dst[i] = (double)results[o][i];
        continue;
      }
      for (int64_t i = 0; i < n; ++i) {
        float v = (float)results[o][i];
        switch (s.dtype) {
          case F32: static_cast<float*>(outputs[o])[i] = v; break;
          case BF16: static_cast<uint16_t*>(outputs[o])[i] = to_bf16(v); break;
          case F16: static_cast<uint16_t*>(outputs[o])[i] = to_f16(v); break;
          case I8: fail("int8 outputs are unsupported");
        }
      }
    }
  }
};

thread_local std::string g_err;

}  // namespace

extern "C" {

// Evaluate `ir` on host buffers.  mode 0: storage dtypes, float32 arithmetic
// with per-op rounding.  mode 1: every buffer is double, binary64 arithmetic.
// Returns 0 on success, -1 with a message (oracle_error) otherwise.
int oracle_run(const char* ir, const void* const* inputs, int n_in, void* const* outputs, int n_out, int mode) {
  try {
    Prog p = parse(ir);
    if ((int)p.inputs.size() != n_in) fail("input count differs from the program signature");
    if ((int)p.outputs.size() != n_out) fail("output count differs from the program signature");
    if (mode == 0) {
      Interp<float> it(p, false);
      it.run(inputs, outputs);
    } else {
      Interp<double> it(p, true);
      it.run(inputs, outputs);
    }
    return 0;
  } catch (const std::exception& e) {
    g_err = e.what();
    return -1;
  }
}

const char* oracle_error(void) { return g_err.c_str(); }

// Threads the oracle's parallel loops use.
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// Set the thread count of later parallel loops (n >= 1).  Results do not
// depend on it: every output is computed by one thread in a fixed order.
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

void oracle_round_bf16(const float* x, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = to_bf16(x[i]);
}

void oracle_round_f16(const float* x, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = to_f16(x[i]);
}

// Fill all 2^32 float32 bit patterns in [lo, lo+n) and count rounding
// disagreements against caller-supplied expected patterns is done in Python;
// this helper generates the inputs quickly.
void oracle_iota_bits(uint32_t lo, uint32_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = lo + (uint32_t)i;
}

}  // extern "C"
