// Host-side program representation and scheduler interfaces of libtk.
#pragma once
#include <cstdint>
#include <map>
#include <set>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/tk.h"
#include "plan.h"

namespace tk {

// A failure with the status code the C ABI returns.
struct Error : std::runtime_error {
  tk_status code;
  Error(tk_status c, const std::string& m) : std::runtime_error("tk: " + m), code(c) {}
};
[[noreturn]] inline void raise(tk_status c, const std::string& m) { throw Error(c, m); }

int dtype_size(uint8_t dt);
const char* dtype_name(uint8_t dt);

// ------------------------------------------------------------------- IR --

struct Spec {
  std::string buf;
  uint8_t dtype = tkplan::DT_F32;
  std::vector<int64_t> shape, strides;
  int64_t offset = 0;
  int64_t numel() const;
  bool contiguous() const;  // size-1 dims may carry any stride
};

struct Arg {
  bool scalar = false;
  float value = 0.0f;
  Spec spec;
};

enum OpClass { OC_POINTWISE, OC_MM, OC_MM_Q8, OC_REDUCE };

struct Op {
  std::string name, opcode;
  Spec out;
  std::vector<Arg> args;
  std::map<std::string, float> attrs;
  bool dims_all = true;
  std::vector<int64_t> dims;
  OpClass cls = OC_POINTWISE;
  float attr(const char* k, float dflt) const {
    auto it = attrs.find(k);
    return it == attrs.end() ? dflt : it->second;
  }
  // Contraction operand indices (A, B [, S]); bias is args[0] for addmm forms.
  bool has_bias() const { return opcode == "addmm" || opcode == "addmm_q8"; }
  const Spec& A() const { return args[has_bias() ? 1 : 0].spec; }
  const Spec& B() const { return args[has_bias() ? 2 : 1].spec; }
  const Spec& S() const { return args[has_bias() ? 3 : 2].spec; }
};

struct Program {
  std::vector<Spec> inputs;
  std::vector<Op> ops;
  std::vector<Spec> outputs;
  std::map<int, int> inplace;  // output slot -> input index
};

Program parse_program(const std::string& text);
void validate_program(const Program& p);

// ------------------------------------------------------------- schedule --

struct Options {
  int blocks_per_cu = 1;
  int max_blocks = 0;
  bool fuse_pointwise = true;
  bool fuse_epilogues = true;
  bool inline_input_casts = true;
  bool split_k_gemv = true;
  bool fuse_updates = true;
  bool barrier_every_op = false;
  int num_cus = 256;
  int gemm_split_k = 0;
  int launch_mode = 0;  // 0 cooperative, 1 ordinary launch of a co-resident grid
  int gemm_tile = 0;    // 0 automatic, 1 force 128x128, 2 force 64x64
  bool fast_epilogue = true;  // contraction epilogues may run as register programs, column sums read directly
  int colsum_fusion = 0;      // 0 where it saves a round of items, 1 wherever legal, -1 never
};

// Compiled plan: device bytes plus host-side description for queries/dumps.
struct Plan {
  std::vector<uint8_t> bytes;  // DHeader | stages | tasks | views | instructions
  uint64_t workspace_bytes = 0;
  int n_in = 0, n_out = 0;
  int ws_base = 0;
  int n_stages = 0;
  int max_items = 0;
  tk_stats stats{};
  std::string dump;
  // per input: index in program; per output: shape/dtype for allocation
  std::vector<Spec> inputs, outputs;
  std::map<int, int> inplace;
};

Plan schedule_program(const Program& p, const Options& o);

}  // namespace tk
