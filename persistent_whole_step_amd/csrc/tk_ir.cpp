// Parsing and validation of `tkir 1` programs.
//
// Validation follows the diagnostics of the trainkernel generator
// (codegen.py: `_literal`, `generate` and `_Generator.generate`, `operand`,
// `point_expr`, `emit_reduction`, `emit_mm`): non-finite scalars, unsupported
// dtypes and operations, negative shapes/strides and bad identifiers,
// broadcast rank/dimension errors, a non-scalar pow exponent, reduction and
// matrix shape errors, non-contiguous computed values, and the in-place map
// rules of `generate`.
#include <cctype>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <sstream>

#include "tk_internal.hpp"

namespace tk {

using namespace tkplan;

int dtype_size(uint8_t dt) {
  switch (dt) {
    case DT_F32: return 4;
    case DT_F16:
    case DT_BF16: return 2;
    case DT_I8: return 1;
  }
  return 0;
}

const char* dtype_name(uint8_t dt) {
  switch (dt) {
    case DT_F32: return "f32";
    case DT_F16: return "f16";
    case DT_BF16: return "bf16";
    case DT_I8: return "i8";
  }
  return "?";
}

int64_t Spec::numel() const {
  int64_t n = 1;
  for (auto d : shape) n *= d;
  return n;
}

bool Spec::contiguous() const {
  int64_t expect = 1;
  for (size_t i = shape.size(); i-- > 0;) {
    if (shape[i] != 1 && strides[i] != expect) return false;
    expect *= shape[i];
  }
  return true;
}

namespace {

std::vector<std::string> split(const std::string& s, char sep) {
  std::vector<std::string> out;
  size_t pos = 0;
  for (;;) {
    size_t n = s.find(sep, pos);
    out.push_back(s.substr(pos, n == std::string::npos ? std::string::npos : n - pos));
    if (n == std::string::npos) break;
    pos = n + 1;
  }
  return out;
}

int64_t to_int(const std::string& s) {
  if (s.empty()) raise(TK_E_PARSE, "empty integer");
  char* end = nullptr;
  long long v = std::strtoll(s.c_str(), &end, 10);
  if (*end) raise(TK_E_PARSE, "bad integer '" + s + "'");
  return v;
}

uint8_t to_dtype(const std::string& s) {
  if (s == "f32") return DT_F32;
  if (s == "f16") return DT_F16;
  if (s == "bf16") return DT_BF16;
  if (s == "i8") return DT_I8;
  raise(TK_E_UNSUPPORTED, "unsupported dtype " + s);
}

std::vector<int64_t> to_dims(const std::string& s) {
  std::vector<int64_t> v;
  if (s == "-") return v;
  for (auto& part : split(s, 'x')) v.push_back(to_int(part));
  return v;
}

float to_scalar(const std::string& s) {
  if (s.size() < 2 || s[0] != '#') raise(TK_E_PARSE, "bad scalar '" + s + "'");
  char* end = nullptr;
  double v = std::strtod(s.c_str() + 1, &end);
  if (*end) raise(TK_E_PARSE, "bad scalar '" + s + "'");
  float f = (float)v;
  if (!std::isfinite(v) || !std::isfinite(f)) raise(TK_E_ARG, "non-finite scalar constants are unsupported");
  if ((double)f != v) raise(TK_E_PARSE, "scalar is not a float32 value: " + s);
  return f;
}

bool valid_ident(const std::string& s) {
  if (s.empty() || !(std::isalpha((unsigned char)s[0]) || s[0] == '_')) return false;
  for (char c : s)
    if (!(std::isalnum((unsigned char)c) || c == '_')) return false;
  return true;
}

Spec to_spec(const std::string& s) {
  auto f = split(s, ':');
  if (f.size() != 5) raise(TK_E_PARSE, "bad tensor spec '" + s + "'");
  Spec v;
  v.buf = f[0];
  v.dtype = to_dtype(f[1]);
  v.shape = to_dims(f[2]);
  v.strides = to_dims(f[3]);
  v.offset = to_int(f[4]);
  return v;
}

void check_spec(const Spec& s) {
  if (!valid_ident(s.buf)) raise(TK_E_ARG, "invalid buffer identifier '" + s.buf + "'");
  if (s.shape.size() != s.strides.size()) raise(TK_E_SHAPE, "invalid static shape or stride: rank mismatch in " + s.buf);
  if (s.shape.size() > 8) raise(TK_E_UNSUPPORTED, "rank above 8 in " + s.buf);
  for (auto d : s.shape)
    if (d < 0) raise(TK_E_SHAPE, "invalid static shape or stride in " + s.buf);
  for (auto d : s.strides)
    if (d < 0) raise(TK_E_STRIDE, "invalid static shape or stride in " + s.buf);
  if (s.offset < 0) raise(TK_E_STRIDE, "negative offset in " + s.buf);
  if (s.numel() > (int64_t)0x7fffffff) raise(TK_E_UNSUPPORTED, "tensor above 2^31 elements: " + s.buf);
  // element indices are 32-bit on the device
  if (s.numel() > 0) {
    int64_t hi = s.offset;
    for (size_t i = 0; i < s.shape.size(); ++i) {
      if (s.strides[i] > (int64_t)0x7fffffff) raise(TK_E_UNSUPPORTED, "stride above 2^31 elements in " + s.buf);
      hi += (s.shape[i] - 1) * s.strides[i];
      if (hi > (int64_t)0x7fffffff) raise(TK_E_UNSUPPORTED, "view addresses beyond 2^31 elements: " + s.buf);
    }
  }
}

// Largest element index a view can address (-1 when empty).
int64_t max_index(const Spec& s) {
  if (s.numel() == 0) return -1;
  int64_t hi = s.offset;
  for (size_t i = 0; i < s.shape.size(); ++i) hi += (s.shape[i] - 1) * s.strides[i];
  return hi;
}

}  // namespace

Program parse_program(const std::string& text) {
  Program p;
  std::istringstream in(text);
  std::string line;
  bool header = false, ended = false;
  while (std::getline(in, line)) {
    auto c = line.find(';');
    if (c != std::string::npos) line.resize(c);
    std::istringstream ls(line);
    std::vector<std::string> tok;
    for (std::string t; ls >> t;) tok.push_back(t);
    if (tok.empty()) continue;
    if (!header) {
      if (tok.size() != 2 || tok[0] != "tkir" || tok[1] != "1") raise(TK_E_PARSE, "missing 'tkir 1' header");
      header = true;
      continue;
    }
    if (ended) raise(TK_E_PARSE, "text after 'end'");
    const std::string& kw = tok[0];
    if (kw == "in") {
      if (tok.size() != 6) raise(TK_E_PARSE, "bad 'in' statement");
      Spec s;
      s.buf = tok[1];
      s.dtype = to_dtype(tok[2]);
      s.shape = to_dims(tok[3]);
      s.strides = to_dims(tok[4]);
      s.offset = to_int(tok[5]);
      p.inputs.push_back(s);
    } else if (kw == "op") {
      if (tok.size() < 4) raise(TK_E_PARSE, "bad 'op' statement");
      Op op;
      op.name = tok[1];
      op.opcode = tok[2];
      op.out = to_spec(tok[3]);
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
              if (!val.empty())
                for (auto& d : split(val, ',')) op.dims.push_back(to_int(d));
            }
          } else if (key == "alpha" || key == "beta" || key == "threshold" || key == "value" || key == "exponent" ||
                     key == "xq") {
            op.attrs[key] = to_scalar(val);
          } else {
            raise(TK_E_PARSE, "unknown attribute '" + key + "'");
          }
        } else if (a[0] == '#') {
          Arg g;
          g.scalar = true;
          g.value = to_scalar(a);
          op.args.push_back(g);
        } else {
          Arg g;
          g.spec = to_spec(a);
          op.args.push_back(g);
        }
      }
      p.ops.push_back(op);
    } else if (kw == "out") {
      if (tok.size() != 2) raise(TK_E_PARSE, "bad 'out' statement");
      p.outputs.push_back(to_spec(tok[1]));
    } else if (kw == "inplace") {
      if (tok.size() != 3) raise(TK_E_PARSE, "bad 'inplace' statement");
      int slot = (int)to_int(tok[1]), idx = (int)to_int(tok[2]);
      if (p.inplace.count(slot)) raise(TK_E_ARG, "in-place slot declared twice");
      p.inplace[slot] = idx;
    } else if (kw == "end") {
      ended = true;
    } else {
      raise(TK_E_PARSE, "unknown statement '" + kw + "'");
    }
  }
  if (!header || !ended) raise(TK_E_PARSE, "incomplete program text (missing header or 'end')");
  return p;
}

void validate_program(const Program& p) {
  std::map<std::string, const Spec*> defined;  // buffer -> defining spec (input or op output)
  std::map<std::string, bool> is_input;
  for (auto& s : p.inputs) {
    check_spec(s);
    if (defined.count(s.buf)) raise(TK_E_ARG, "buffer '" + s.buf + "' is defined twice");
    defined[s.buf] = &s;
    is_input[s.buf] = true;
  }
  auto check_operand = [&](const Spec& v, const char* what) {
    check_spec(v);
    auto it = defined.find(v.buf);
    if (it == defined.end()) raise(TK_E_ARG, std::string(what) + " '" + v.buf + "' is not defined before use");
    if (v.dtype != it->second->dtype)
      raise(TK_E_DTYPE, "view of '" + v.buf + "' has dtype " + dtype_name(v.dtype) + ", buffer has " +
                            dtype_name(it->second->dtype));
    // The view must stay within its buffer's addressable extent.
    const Spec& src = *it->second;
    int64_t hi = max_index(v), cap = is_input[v.buf] ? max_index(src) : src.numel() - 1;
    if (hi > cap) raise(TK_E_SHAPE, "view of '" + v.buf + "' exceeds its buffer's extent");
  };
  auto check_broadcast = [&](const Spec& v, const std::vector<int64_t>& out) {
    if (v.shape.size() > out.size()) raise(TK_E_SHAPE, "invalid broadcast rank");
    size_t off = out.size() - v.shape.size();
    for (size_t i = 0; i < v.shape.size(); ++i)
      if (v.shape[i] != 1 && v.shape[i] != out[off + i]) raise(TK_E_SHAPE, "incompatible broadcast dimensions");
  };
  static const std::set<std::string> pointwise = {"add", "sub", "mul", "div", "neg", "relu", "pow",
                                                  "threshold_backward", "full", "cast", "sqrt"};
  for (auto& op : p.ops) {
    check_spec(op.out);
    if (op.out.dtype == DT_I8) raise(TK_E_DTYPE, "operations produce float values only: " + op.name);
    if (op.out.offset != 0 || !op.out.contiguous())
      raise(TK_E_STRIDE, "materialized output must be contiguous: " + op.name);
    for (auto& a : op.args)
      if (!a.scalar) check_operand(a.spec, "operand");
    const std::string& c = op.opcode;
    const size_t n = op.args.size();
    if (op.attrs.count("xq") && c != "mm_q8" && c != "addmm_q8") raise(TK_E_ARG, "xq applies to the q8 products only");
    if (pointwise.count(c)) {
      const_cast<Op&>(op).cls = OC_POINTWISE;
      for (auto& a : op.args)
        if (!a.scalar) check_broadcast(a.spec, op.out.shape);
      if ((c == "neg" || c == "relu" || c == "cast" || c == "sqrt") && n != 1) raise(TK_E_ARG, c + " takes one operand");
      if ((c == "add" || c == "sub" || c == "mul" || c == "div" || c == "threshold_backward") && n != 2)
        raise(TK_E_ARG, c + " takes two operands");
      if (c == "pow") {
        if (n < 1 || n > 2) raise(TK_E_ARG, "pow takes one operand and an exponent");
        if (n == 2 && !op.args[1].scalar) raise(TK_E_ARG, "pow exponent must be a scalar");
      }
      if (c == "full" && n > 1) raise(TK_E_ARG, "full takes at most one scalar");
      if (c == "full" && n == 1 && !op.args[0].scalar && !op.attrs.count("value"))
        raise(TK_E_ARG, "full takes a scalar value");
    } else if (c == "mm" || c == "addmm" || c == "mm_q8" || c == "addmm_q8") {
      const bool q8 = c == "mm_q8" || c == "addmm_q8";
      const_cast<Op&>(op).cls = q8 ? OC_MM_Q8 : OC_MM;
      const size_t want = (op.has_bias() ? 1 : 0) + (q8 ? 3 : 2);
      if (n != want) raise(TK_E_ARG, "wrong operand count for " + c);
      for (auto& a : op.args)
        if (a.scalar) raise(TK_E_UNSUPPORTED, "matrix operands must be tensors");
      const Spec &A = op.A(), &B = op.B();
      if (A.shape.size() != 2 || B.shape.size() != 2) raise(TK_E_SHAPE, "mm requires compatible rank-two tensors");
      int64_t m = A.shape[0], k = A.shape[1], nn;
      if (q8) {
        if (B.dtype != DT_I8 || B.shape[1] != k) raise(TK_E_SHAPE, "q8 weight must be int8 [n, k]");
        nn = B.shape[0];
        const Spec& S = op.S();
        if (S.dtype != DT_F32 || S.shape.size() != 2 || S.shape[0] != nn || S.shape[1] != (k + 31) / 32)
          raise(TK_E_SHAPE, "q8 scales must be float32 [n, ceil(k/32)]");
        if (A.dtype == DT_I8) raise(TK_E_DTYPE, "activations must be float");
        if (op.attrs.count("xq") && op.attrs.at("xq") != 0.0f && op.attrs.at("xq") != 1.0f)
          raise(TK_E_ARG, "xq must be 0 or 1");
      } else {
        if (B.shape[0] != k) raise(TK_E_SHAPE, "mm requires compatible rank-two tensors");
        if (A.dtype == DT_I8 || B.dtype == DT_I8) raise(TK_E_DTYPE, "int8 operands need the q8 form");
        nn = B.shape[1];
      }
      if (op.out.shape.size() != 2 || op.out.shape[0] != m || op.out.shape[1] != nn)
        raise(TK_E_SHAPE, "matrix output shape does not match its inputs");
      if (op.has_bias()) check_broadcast(op.args[0].spec, op.out.shape);
    } else if (c == "sum" || c == "mean") {
      const_cast<Op&>(op).cls = OC_REDUCE;
      if (n != 1 || op.args[0].scalar) raise(TK_E_ARG, "reduction requires a tensor");
      const Spec& x = op.args[0].spec;
      const int64_t r = (int64_t)x.shape.size();
      if (!op.dims_all && r == 0 && !op.dims.empty()) raise(TK_E_SHAPE, "cannot reduce a rank-zero tensor over dims");
      std::set<int64_t> red;
      if (op.dims_all) {
        for (int64_t d = 0; d < r; ++d) red.insert(d);
      } else {
        for (auto d : op.dims) red.insert(((d % r) + r) % r);
      }
      int64_t kept = 1;
      for (int64_t d = 0; d < r; ++d)
        if (!red.count(d)) kept *= x.shape[d];
      if (op.out.numel() != kept) raise(TK_E_SHAPE, "reduction output shape does not match its axes");
    } else {
      raise(TK_E_UNSUPPORTED, "unsupported operation " + c);
    }
    if (!valid_ident(op.out.buf)) raise(TK_E_ARG, "invalid buffer identifier '" + op.out.buf + "'");
    if (defined.count(op.out.buf)) raise(TK_E_ARG, "buffer '" + op.out.buf + "' is defined twice");
    defined[op.out.buf] = &op.out;
    is_input[op.out.buf] = false;
  }
  for (auto& o : p.outputs) {
    check_spec(o);
    auto it = defined.find(o.buf);
    if (it == defined.end()) raise(TK_E_ARG, "output '" + o.buf + "' is not defined");
    if (o.dtype == DT_I8) raise(TK_E_DTYPE, "int8 outputs are unsupported");
    int64_t hi = max_index(o), cap = is_input[o.buf] ? max_index(*it->second) : it->second->numel() - 1;
    if (hi > cap) raise(TK_E_SHAPE, "output view of '" + o.buf + "' exceeds its buffer's extent");
  }
  // In-place map (codegen.py `generate`): valid indices, distinct targets,
  // same shape and dtype as a contiguous input, and a computed value.
  std::set<int> targets;
  for (auto& kv : p.inplace) {
    int slot = kv.first, idx = kv.second;
    if (slot < 0 || slot >= (int)p.outputs.size() || idx < 0 || idx >= (int)p.inputs.size())
      raise(TK_E_ARG, "invalid inplace output/input index");
    if (!targets.insert(idx).second) raise(TK_E_ARG, "inplace outputs must target distinct inputs");
    const Spec &o = p.outputs[slot], &in = p.inputs[idx];
    if (o.shape != in.shape || o.dtype != in.dtype || !in.contiguous() || in.offset != 0)
      raise(TK_E_SHAPE, "inplace output must match a contiguous input shape and dtype");
    if (is_input[o.buf]) raise(TK_E_ARG, "inplace outputs must be computed values, not input views");
  }
}

}  // namespace tk
