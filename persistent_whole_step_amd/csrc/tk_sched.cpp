// Scheduler: program -> stages of device tasks.
//
// The decisions follow the trainkernel generator (codegen.py, `_Generator`):
//  * epilogue fusion, pass 1: a non-returned contraction followed by a chain of
//    single-use, shape-preserving pointwise ops is replaced by one tile task
//    writing the chain's last value (identity-viewed chain links, contiguous
//    external operands produced before the contraction);
//  * pass 2 ("side epilogues"): the tile also writes returned pointwise
//    descendants of a kept (or discarded) root;
//  * inlining of single-use pointwise values and of casts of inputs;
//  * the direct in-place commit proof and staged (transactional) commits;
//  * output bindings, workspace reuse after the last reader, hazard-driven
//    barrier placement (read/write region overlap), grid sizing.
// Additions of this design, all value-preserving:
//  * ops are levelled (1 + the latest stage they depend on, including
//    write-after-read on in-place targets), so independent ops share a stage;
//  * pass 3 folds a proven-direct in-place pointwise update (e.g. SGD) into the
//    tile of the contraction that produces its only non-input operand, when
//    that contraction reads nothing of the target;
//  * workspace values keep their storage dtype (2-byte bf16/f16) instead of
//    float32, with identical values;
//  * long reductions and split-K contractions are two stages with fp32
//    partials combined in a fixed order, covering every element.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <sstream>

#include "tk_internal.hpp"

namespace tk {

using namespace tkplan;

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

static const char* kind_name(uint8_t k) {
  switch (k) {
    case T_EW: return "ew";
    case T_GEMM_MFMA: return "gemm_mfma";
    case T_GEMM_SIMT: return "gemm_simt";
    case T_GEMM_REDUCE: return "gemm_splitk_reduce";
    case T_GEMV_Q8: return "gemv_q8";
    case T_GEMV: return "gemv";
    case T_RED_ROWS: return "reduce_rows";
    case T_RED_COLS: return "reduce_cols";
    case T_RED_FINAL: return "reduce_final";
  }
  return "?";
}

// Where a materialized value lives.
struct Loc {
  int base = -1;        // base slot
  int64_t offset = 0;   // elements
  uint8_t dtype = DT_F32;
  bool valid() const { return base >= 0; }
};

// Expression tree over one op's iteration space.
struct Node {
  enum Kind { LEAF, SCALAR, SLOT, OP } kind = LEAF;
  int view = -1;       // LEAF: index into the task's view table
  float value = 0;     // SCALAR
  int slot = -1;       // SLOT
  int op = -1;         // OP: program op index
  std::vector<Node> kids;
};

struct Entry {            // one scheduled (materialized) unit
  int op = -1;            // program op index (the contraction for fused tiles)
  std::vector<int> chain; // pass 1 / pass 3 chain ops
  std::vector<int> side;  // pass 2 descendants
  bool discard_root = false;
  bool update = false;    // pass 3
  int kind = 0;           // 0 op, 1 output copy, 2 staged commit
  int slot = -1;          // output slot for copies/commits
  int level = 0;
  bool two_phase = false;
  int avail() const { return level + (two_phase ? 1 : 0); }
  std::vector<std::string> reads_vals;    // materialized values read
  std::set<std::string> reads_inputs;     // input buffers read (through inline)
  std::set<std::string> writes_vals;      // values written
  std::vector<int> writes_inputs;         // input indices written (direct in-place / commit)
  int order = 0;
};

struct Builder {
  const Program& P;
  const Options& O;
  int n_in, n_out, ws_base;
  std::map<std::string, int> input_idx, producer;
  std::map<std::string, std::vector<int>> users;  // with multiplicity (one per operand reference)
  std::map<std::string, int> refcount;
  std::set<std::string> output_bufs;
  std::map<std::string, int> output_count;
  std::set<std::string> aliased;   // declared in-place output buffers

  std::map<int, Entry> fused;      // by contraction op index
  std::set<int> skip;              // ops computed inside a fused tile
  std::set<int> inlined;
  std::set<std::string> inlined_bufs;
  std::vector<Entry> sched;
  std::map<int, int> direct;       // output slot -> input index
  std::map<int, int> colsum_of;    // contraction entry -> column reduction entry it also runs (F_BSUM)
  std::map<int, int> colsum_host;  // that reduction entry -> the contraction entry
  std::map<std::string, int> bound;  // value -> output slot written directly
  std::map<std::string, Loc> loc;    // value -> storage
  std::map<std::string, uint64_t> arena_off;  // value -> byte offset in arena

  // device tables
  std::vector<DView> views;
  std::vector<DIns> ins;
  std::vector<std::vector<DTask>> stage_tasks;
  std::vector<std::vector<std::string>> stage_desc;
  std::map<int, uint64_t> scratch_off;  // sched index -> scratch byte offset
  std::map<int, uint64_t> scratch_bytes;
  uint64_t arena_bytes = 0;
  tk_stats st{};

  Builder(const Program& p, const Options& o) : P(p), O(o) {
    n_in = (int)p.inputs.size();
    n_out = (int)p.outputs.size();
    ws_base = n_in + n_out;
    if (ws_base + 1 > kMaxBases) raise(TK_E_UNSUPPORTED, "too many inputs and outputs for one launch");
    for (int i = 0; i < n_in; ++i) input_idx[p.inputs[i].buf] = i;
    for (int j = 0; j < (int)p.ops.size(); ++j) {
      producer[p.ops[j].out.buf] = j;
      for (auto& a : p.ops[j].args)
        if (!a.scalar) {
          users[a.spec.buf].push_back(j);
          refcount[a.spec.buf]++;
        }
    }
    for (auto& o2 : p.outputs) {
      output_bufs.insert(o2.buf);
      output_count[o2.buf]++;
    }
    for (auto& kv : p.inplace) aliased.insert(p.outputs[kv.first].buf);
  }

  const Op& op(int j) const { return P.ops[j]; }
  bool is_input(const std::string& b) const { return input_idx.count(b) != 0; }
  int prod(const std::string& b) const {
    auto it = producer.find(b);
    return it == producer.end() ? -1 : it->second;
  }
  bool is_contraction(int j) const { return op(j).cls == OC_MM || op(j).cls == OC_MM_Q8; }
  static bool identity_view(const Spec& s, const std::vector<int64_t>& shape) {
    return s.shape == shape && s.offset == 0 && s.contiguous();
  }

  // ------------------------------------------------------------ fusion --
  void pass1() {
    for (int mi = 0; mi < (int)P.ops.size(); ++mi) {
      const Op& mm = op(mi);
      if (!is_contraction(mi) || output_bufs.count(mm.out.buf)) continue;
      std::vector<int> chain;
      std::string cur = mm.out.buf;
      for (;;) {
        auto uit = users.find(cur);
        if (uit == users.end() || uit->second.size() != 1) break;
        int nj = uit->second[0];
        const Op& nx = op(nj);
        if (nx.cls != OC_POINTWISE || output_bufs.count(nx.out.buf)) break;
        const std::vector<int64_t>& cur_shape = op(prod(cur)).out.shape;
        bool ok = true;
        for (auto& a : nx.args)
          if (!a.scalar && a.spec.buf == cur && !identity_view(a.spec, cur_shape)) ok = false;
        if (!ok) break;
        chain.push_back(nj);
        cur = nx.out.buf;
      }
      if (chain.empty()) continue;
      bool safe = true;
      std::set<std::string> chain_bufs = {mm.out.buf};
      for (int c : chain) chain_bufs.insert(op(c).out.buf);
      for (int c : chain) {
        if (op(c).out.shape != mm.out.shape) safe = false;
        for (auto& a : op(c).args) {
          if (a.scalar || chain_bufs.count(a.spec.buf)) continue;
          if (a.spec.offset != 0 || !a.spec.contiguous()) safe = false;
          if (prod(a.spec.buf) >= mi) safe = false;
        }
      }
      if (!safe) continue;
      Entry e;
      e.op = mi;
      e.chain = chain;
      fused[mi] = e;
      for (int c : chain) skip.insert(c);
    }
  }

  // A value computed by pointwise ops from inputs and scalars alone: any task
  // can evaluate (or read) it, whatever its place in program order.
  bool input_pure(const std::string& b) const {
    if (is_input(b)) return true;
    const int j = prod(b);
    if (j < 0 || op(j).cls != OC_POINTWISE || output_bufs.count(b)) return false;
    for (auto& a : op(j).args)
      if (!a.scalar && !input_pure(a.spec.buf)) return false;
    return true;
  }

  // Whether a view can be read over the flattened output space of a
  // reduction root (rank other than one): the root's own shape, contiguous,
  // or one element broadcast.
  static bool flattenable(const Spec& s, const std::vector<int64_t>& shape) {
    return (s.shape == shape && s.contiguous()) || s.numel() == 1 ||
           std::all_of(s.strides.begin(), s.strides.end(), [](int64_t v) { return v == 0; });
  }

  // Pass 2 ("side epilogues"): a contraction tile or a reduction's finishing
  // program also evaluates pointwise descendants of its result over the same
  // index space and writes those that are returned or read elsewhere.
  // Additions of this design: a derived value read by an op outside the tile
  // is written too (to its usual home), so the pointwise stage that would
  // recompute it disappears; reductions are roots as well as contractions;
  // returned in-place values (parameter and optimizer-state updates) may be
  // descendants, committed directly when the in-place proof holds; operands
  // that are pure functions of inputs may come later in program order.
  void pass2() {
    for (int mi = 0; mi < (int)P.ops.size(); ++mi) {
      const Op& mm = op(mi);
      const bool red = mm.cls == OC_REDUCE;
      if ((!is_contraction(mi) && !red) || skip.count(mi)) continue;
      // a pass-1 chain is extended when more descendants can join it (the
      // chain's links become side ops)
      const bool from_pass1 = fused.count(mi) && !fused[mi].chain.empty() && fused[mi].side.empty();
      if (fused.count(mi) && !from_pass1) continue;
      const std::vector<int64_t>& rshape = mm.out.shape;
      const bool flat = red && rshape.size() != 1;
      std::set<std::string> known = {mm.out.buf};
      std::vector<int> chain;
      std::set<int> seeded;
      if (from_pass1)
        for (int c : fused[mi].chain) {
          chain.push_back(c);
          seeded.insert(c);
          known.insert(op(c).out.buf);
        }
      for (int j = mi + 1; j < (int)P.ops.size(); ++j) {
        const Op& nx = op(j);
        if (seeded.count(j)) continue;
        if (nx.cls != OC_POINTWISE || skip.count(j)) continue;
        bool touches = false;
        for (auto& a : nx.args)
          if (!a.scalar && known.count(a.spec.buf)) touches = true;
        if (!touches) continue;
        if (nx.out.shape != rshape) continue;
        if (aliased.count(nx.out.buf) && !O.fuse_updates) continue;
        bool ok = true;
        for (auto& a : nx.args) {
          if (a.scalar) continue;
          if (known.count(a.spec.buf)) {
            if (!identity_view(a.spec, rshape)) ok = false;
          } else {
            if (prod(a.spec.buf) >= mi && !input_pure(a.spec.buf)) ok = false;
            if (flat && !flattenable(a.spec, rshape)) ok = false;
          }
        }
        if (!ok) continue;
        chain.push_back(j);
        known.insert(nx.out.buf);
      }
      if (from_pass1 && chain.size() == seeded.size()) continue;  // nothing to add
      std::sort(chain.begin(), chain.end());
      std::set<std::string> derived = known;
      derived.erase(mm.out.buf);
      std::set<std::string> returned;
      for (auto& d : derived)
        if (output_bufs.count(d)) returned.insert(d);
      std::set<std::string> chain_outs;
      for (int c : chain) chain_outs.insert(op(c).out.buf);
      std::set<std::string> escaping;
      for (auto& d : derived) {
        if (returned.count(d)) continue;
        for (int u : users[d])
          if (!chain_outs.count(op(u).out.buf)) escaping.insert(d);
      }
      std::set<std::string> needed = returned;
      needed.insert(escaping.begin(), escaping.end());
      for (auto it = chain.rbegin(); it != chain.rend(); ++it)
        if (needed.count(op(*it).out.buf))
          for (auto& a : op(*it).args)
            if (!a.scalar && derived.count(a.spec.buf)) needed.insert(a.spec.buf);
      std::vector<int> kept;
      for (int c : chain)
        if (needed.count(op(c).out.buf)) kept.push_back(c);
      std::set<std::string> dkept;
      for (auto& d : derived)
        if (needed.count(d)) dkept.insert(d);
      if (returned.empty() && escaping.empty()) continue;
      bool ok = true;
      // every reader of a kept value that is neither returned nor stored must
      // be inside the tile
      for (auto& d : dkept) {
        if (returned.count(d) || escaping.count(d)) continue;
        for (int u : users[d])
          if (!dkept.count(op(u).out.buf)) ok = false;
      }
      // returned values must be bindable straight into their output buffer
      // (in-place values are committed directly or staged instead)
      for (auto& r : returned) {
        if (aliased.count(r)) continue;
        bool bindable = false;
        for (int s = 0; s < n_out; ++s) {
          const Spec& o2 = P.outputs[s];
          if (o2.buf != r || P.inplace.count(s)) continue;
          const Spec& pv = op(prod(r)).out;
          if (o2.offset == 0 && o2.shape == pv.shape && o2.contiguous() && o2.dtype == pv.dtype) bindable = true;
        }
        if (!bindable) ok = false;
      }
      if (!ok) continue;
      Entry e;
      e.op = mi;
      e.side = kept;
      bool root_only_chain = !output_bufs.count(mm.out.buf);
      for (int u : users[mm.out.buf])
        if (!dkept.count(op(u).out.buf)) root_only_chain = false;
      e.discard_root = root_only_chain;
      // the side program must fit the machine's slots
      std::set<std::string> ext;
      for (int j = 0; j < (int)P.ops.size(); ++j)
        if (!skip.count(j) && !dkept.count(op(j).out.buf) && inlinable(j)) ext.insert(op(j).out.buf);
      if (!plan_side(e, ext).ok) continue;
      // a replaced pass-1 entry must still compute every link it owned
      bool covers = true;
      for (int c : seeded)
        if (std::find(kept.begin(), kept.end(), c) == kept.end()) covers = false;
      if (!covers) continue;
      fused[mi] = e;
      for (int c : kept) skip.insert(c);
    }
  }

  // ------------------------------------------------------- side programs --
  // A side program runs after the root value (a tile's or a reduction's
  // result) is in the accumulator.  A side value that is not stored and has
  // exactly one reader among the side ops is expanded into that reader's
  // expression; the others are evaluated in program order, stored when
  // written to storage, and held in a slot while later side ops read them.
  struct SidePlan {
    std::vector<int> evals;               // side ops evaluated in turn
    std::set<std::string> expanded;       // side values expanded into their reader
    std::map<std::string, int> slot;      // held value -> slot
    std::vector<uint32_t> busy;           // per eval: slots holding values during it
    std::map<int, int> pos;               // side op -> eval index where its value is computed
    int slots = 0;                        // slots used, temporaries included
    bool ok = true;
  };

  // Temporaries an operand's expression needs (Sethi-Ullman numbering for the
  // accumulator machine); `simple` when it is one load.
  int need_arg(const Arg& a, const std::set<std::string>& held, const std::set<std::string>& expand,
               const std::set<std::string>& inl, bool& simple) const {
    simple = true;
    if (a.scalar || held.count(a.spec.buf)) return 0;
    if (expand.count(a.spec.buf) || inl.count(a.spec.buf)) {
      simple = false;
      return need_op(prod(a.spec.buf), held, expand, inl);
    }
    return 0;
  }
  int need_op(int j, const std::set<std::string>& held, const std::set<std::string>& expand,
              const std::set<std::string>& inl) const {
    const Op& o2 = op(j);
    if (o2.opcode == "full" || o2.args.empty()) return 0;
    bool sx = true, sy = true;
    const int nx = need_arg(o2.args[0], held, expand, inl, sx);
    const bool binary = o2.opcode == "add" || o2.opcode == "sub" || o2.opcode == "mul" || o2.opcode == "div" ||
                        o2.opcode == "threshold_backward";
    if (!binary) return nx;
    const int ny = need_arg(o2.args[1], held, expand, inl, sy);
    if (sy) return nx;
    if (sx) return ny;
    return ny > nx ? std::max(ny, 1 + nx) : std::max(nx, 1 + ny);
  }

  // Held values (root and evaluated side values) an expression reads.
  void held_refs(int j, const std::set<std::string>& expand, const std::set<std::string>& inl,
                 const std::set<std::string>& holdable, std::set<std::string>& out) const {
    for (auto& a : op(j).args) {
      if (a.scalar) continue;
      const std::string& b = a.spec.buf;
      if (holdable.count(b))
        out.insert(b);
      else if (expand.count(b) || inl.count(b))
        held_refs(prod(b), expand, inl, holdable, out);
    }
  }

  SidePlan plan_side(const Entry& e, const std::set<std::string>& inl) const {
    SidePlan sp;
    const std::string root = op(e.op).out.buf;
    std::map<std::string, int> readers;
    for (int c : e.side)
      for (auto& a : op(c).args)
        if (!a.scalar) readers[a.spec.buf]++;
    for (int c : e.side) {
      const std::string& b = op(c).out.buf;
      if (!side_stored(e, c) && readers[b] == 1)
        sp.expanded.insert(b);
      else
        sp.evals.push_back(c);
    }
    std::set<std::string> holdable = {root};
    for (int c : sp.evals) holdable.insert(op(c).out.buf);
    std::map<std::string, int> last_use;
    std::vector<std::set<std::string>> refs(sp.evals.size());
    for (size_t i = 0; i < sp.evals.size(); ++i) {
      held_refs(sp.evals[i], sp.expanded, inl, holdable, refs[i]);
      for (auto& v : refs[i]) last_use[v] = (int)i;
    }
    // where each expanded value is computed: inside its reader's evaluation
    std::function<int(const std::string&)> at = [&](const std::string& b) -> int {
      for (size_t i = 0; i < sp.evals.size(); ++i)
        if (op(sp.evals[i]).out.buf == b) return (int)i;
      for (int c : e.side)
        for (auto& a : op(c).args)
          if (!a.scalar && a.spec.buf == b) return at(op(c).out.buf);
      return (int)sp.evals.size();
    };
    for (int c : e.side) sp.pos[c] = at(op(c).out.buf);
    std::map<int, std::string> live;  // slot -> value
    if (last_use.count(root)) {
      live[0] = root;
      sp.slot[root] = 0;
      sp.slots = 1;
    }
    for (size_t i = 0; i < sp.evals.size(); ++i) {
      std::set<std::string> held;
      uint32_t mask = 0;
      for (auto& kv : live) {
        held.insert(kv.second);
        mask |= 1u << kv.first;
      }
      sp.busy.push_back(mask);
      // temporaries take the lowest free slots: the highest one in use
      int top = 0, need = need_op(sp.evals[i], held, sp.expanded, inl);
      for (int k = 0; need > 0 || (mask >> k); ++k)
        if (mask & (1u << k)) top = k + 1;
        else if (need > 0) { --need; top = k + 1; }
      sp.slots = std::max(sp.slots, top);
      for (auto it = live.begin(); it != live.end();)
        it = last_use[it->second] <= (int)i ? live.erase(it) : std::next(it);
      const std::string& b = op(sp.evals[i]).out.buf;
      if (last_use.count(b) && last_use[b] > (int)i) {
        int s = 0;
        while (live.count(s)) ++s;
        live[s] = b;
        sp.slot[b] = s;
        sp.slots = std::max(sp.slots, s + 1);
      }
    }
    sp.ok = sp.slots <= kMaxSlots;
    return sp;
  }

  // ---------------------------------------------------------- inlining --
  // Whether a pointwise value may be recomputed inside its one reader (or,
  // for casts of inputs, inside every reader).
  bool inlinable(int j) const {
    const Op& o2 = op(j);
    if (!O.fuse_pointwise || o2.cls != OC_POINTWISE) return false;
    if (output_bufs.count(o2.out.buf)) return false;
    bool input_cast = O.inline_input_casts && o2.opcode == "cast" && !o2.args[0].scalar && is_input(o2.args[0].spec.buf);
    auto rc = refcount.find(o2.out.buf);
    if (!((rc != refcount.end() && rc->second == 1) || input_cast)) return false;
    // Readers must see the value through an identity view and must not be
    // contraction operands (the matrix loaders read storage).
    auto us = users.find(o2.out.buf);
    if (us == users.end()) return true;
    for (int u : us->second) {
      const Op& uo = op(u);
      for (size_t ai = 0; ai < uo.args.size(); ++ai) {
        const Arg& a = uo.args[ai];
        if (a.scalar || a.spec.buf != o2.out.buf) continue;
        if (!identity_view(a.spec, o2.out.shape)) return false;
        if (uo.cls == OC_MM || uo.cls == OC_MM_Q8)
          if (!(uo.has_bias() && ai == 0)) return false;
      }
    }
    return true;
  }

  void choose_inline() {
    for (int j = 0; j < (int)P.ops.size(); ++j) {
      if (skip.count(j) || !inlinable(j)) continue;
      inlined.insert(j);
      inlined_bufs.insert(op(j).out.buf);
    }
  }

  // Which caller inputs a value's elements are computed from, through the
  // producers inlined into its readers, and whether element i of the value
  // depends on each such input only through its element i.  Filled once the
  // inlining is fixed (producers precede their users in program order).
  struct InputUse {
    std::map<std::string, bool> aligned;  // input -> read element for element on every path
  };
  std::map<std::string, InputUse> input_use;

  void build_input_use() {
    input_use.clear();
    for (auto& in : P.inputs) input_use[in.buf].aligned[in.buf] = true;
    for (int j = 0; j < (int)P.ops.size(); ++j) {
      const Op& o2 = op(j);
      if (!inlined_bufs.count(o2.out.buf)) continue;
      InputUse u;
      for (auto& a : o2.args) {
        if (a.scalar) continue;
        auto it = input_use.find(a.spec.buf);
        if (it == input_use.end()) continue;  // a materialised value: no input behind it
        const bool hop = identity_view(a.spec, o2.out.shape);
        for (auto& kv : it->second.aligned) {
          auto ins = u.aligned.emplace(kv.first, true).first;
          ins->second = ins->second && hop && kv.second;
        }
      }
      input_use[o2.out.buf] = u;
    }
  }
  // Whether reading view s reads any element of input buffer target.
  bool reads_input(const Spec& s, const std::string& target) const {
    auto it = input_use.find(s.buf);
    return it != input_use.end() && it->second.aligned.count(target) != 0;
  }
  // Caller inputs read through view s.
  std::set<std::string> inputs_read(const Spec& s) const {
    std::set<std::string> r;
    auto it = input_use.find(s.buf);
    if (it != input_use.end())
      for (auto& kv : it->second.aligned) r.insert(kv.first);
    return r;
  }
  // Whether every read of target through view s, evaluated at element i of an
  // iteration space of the given shape, reads the target's element i: the view
  // and every inlined step below it are whole, contiguous and of that shape.
  bool reads_aligned(const Spec& s, const std::string& target, const std::vector<int64_t>& shape) const {
    if (!reads_input(s, target)) return true;
    if (!identity_view(s, shape)) return false;
    if (s.buf == target) return true;
    return op(prod(s.buf)).out.shape == shape && input_use.at(s.buf).aligned.at(target);
  }
  // Materialized values reachable from a view through inlined producers.
  void root_values(const Spec& s, std::vector<std::string>& out) const {
    if (is_input(s.buf)) return;
    if (inlined_bufs.count(s.buf)) {
      for (auto& a : op(prod(s.buf)).args)
        if (!a.scalar) root_values(a.spec, out);
      return;
    }
    out.push_back(s.buf);
  }
  // Ops (by program index) and their operands as read by an entry.
  std::vector<const Arg*> entry_args(const Entry& e) const {
    std::vector<const Arg*> r;
    if (e.kind != 0) return r;
    for (auto& a : op(e.op).args) r.push_back(&a);
    for (int c : e.chain)
      for (auto& a : op(c).args) r.push_back(&a);
    for (int c : e.side)
      for (auto& a : op(c).args) r.push_back(&a);
    return r;
  }
  std::set<std::string> internal_bufs(const Entry& e) const {
    std::set<std::string> s;
    if (e.kind != 0) return s;
    s.insert(op(e.op).out.buf);
    for (int c : e.chain) s.insert(op(c).out.buf);
    for (int c : e.side) s.insert(op(c).out.buf);
    return s;
  }
  std::string final_buf(const Entry& e) const {
    if (!e.chain.empty()) return op(e.chain.back()).out.buf;
    return op(e.op).out.buf;
  }

  // Whether an entry's side ops write a returned in-place value.
  bool writes_aliased(const Entry& e) const {
    for (int c : e.side)
      if (aliased.count(op(c).out.buf)) return true;
    return false;
  }

  void build_schedule() {
    // An entry whose side ops update state in place takes the place of its
    // last side op in program order (after the readers of the old state), as
    // the update it absorbs would have.
    std::map<int, std::vector<Entry>> at;
    for (int j = 0; j < (int)P.ops.size(); ++j) {
      if (fused.count(j)) {
        const Entry& f = fused[j];
        int place = j;
        if (writes_aliased(f))
          for (int c : f.side) place = std::max(place, c);
        at[place].push_back(f);
      } else if (!skip.count(j) && !inlined.count(j)) {
        Entry e;
        e.op = j;
        at[j].push_back(e);
      }
    }
    for (auto& kv : at)
      for (auto& e : kv.second) sched.push_back(e);
    for (size_t i = 0; i < sched.size(); ++i) sched[i].order = (int)i;
  }

  // Whether entry i reads, directly or through other entries, a value that
  // entry w writes.
  bool depends_on(int i, int w) const {
    std::map<std::string, int> writer;
    for (size_t k = 0; k < sched.size(); ++k)
      for (auto& v : written(sched[k])) writer[v] = (int)k;
    std::vector<int> stack = {i};
    std::set<int> seen;
    while (!stack.empty()) {
      const int k = stack.back();
      stack.pop_back();
      if (!seen.insert(k).second) continue;
      const auto internal = internal_bufs(sched[k]);
      for (auto* a : entry_args(sched[k])) {
        if (a->scalar || internal.count(a->spec.buf)) continue;
        std::vector<std::string> rv;
        root_values(a->spec, rv);
        for (auto& v : rv) {
          auto it = writer.find(v);
          if (it == writer.end()) continue;
          if (it->second == w) return true;
          stack.push_back(it->second);
        }
      }
    }
    return false;
  }

  // Whether a side-epilogue value is written to storage: it is returned, or
  // an op outside the tile reads it.
  bool side_stored(const Entry& e, int c) const {
    const std::string& b = op(c).out.buf;
    if (output_bufs.count(b)) return true;
    auto it = users.find(b);
    if (it == users.end()) return false;
    const std::set<std::string> inside = internal_bufs(e);
    for (int u : it->second)
      if (!inside.count(op(u).out.buf)) return true;
    return false;
  }

  // Values an entry writes to storage.
  std::vector<std::string> written(const Entry& e) const {
    std::vector<std::string> w;
    if (e.kind != 0) return w;
    if (!e.side.empty()) {
      if (!e.discard_root) w.push_back(op(e.op).out.buf);
      for (int c : e.side)
        if (side_stored(e, c)) w.push_back(op(c).out.buf);
      return w;
    }
    w.push_back(final_buf(e));
    return w;
  }

  // ----------------------------------------------- direct in-place proof --
  // An in-place output may be written straight into its target input T when
  // no read of T's old contents can observe the new ones.  The reads of T that
  // the write cannot disturb are
  //   (1) reads by entries that finish before the writing entry starts (the
  //       leveling puts every such reader at an earlier stage), and
  //   (2) reads inside the writing entry of element i, made by the thread that
  //       computes element i, before it stores element i.
  // The checks below establish exactly that and nothing stronger.

  // Index of the entry that stores value v, or -1.
  int entry_writing(const std::string& v) const {
    int who = -1;
    for (size_t i = 0; i < sched.size(); ++i)
      for (auto& w : written(sched[i]))
        if (w == v) who = (int)i;
    return who;
  }
  // Whether entry i reads any element of input T (through its operands).
  bool entry_reads_input(int i, const std::string& T) const {
    for (auto* a : entry_args(sched[i]))
      if (!a->scalar && reads_input(a->spec, T)) return true;
    return false;
  }

  // (2) for a plain pointwise entry: every operand reads T element for
  // element over the output's shape.
  bool plain_reads_in_step(const Entry& e, const std::string& T, const std::vector<int64_t>& shape) const {
    for (auto& a : op(e.op).args)
      if (!a.scalar && !reads_aligned(a.spec, T, shape)) return false;
    return true;
  }
  // (2) for a contraction tile whose side op `wop` stores the new T: the
  // contraction's operands (read across rows and columns) never touch T, and
  // every side op reading T reads it element for element and runs no later
  // than `wop` in the tile's per-element program.
  bool tile_reads_in_step(const Entry& e, int wop, const std::string& T, const std::vector<int64_t>& shape) const {
    for (auto& a : op(e.op).args)
      if (!a.scalar && reads_input(a.spec, T)) return false;
    const SidePlan sp = plan_side(e, inlined_bufs);
    for (int c : e.side)
      for (auto& a : op(c).args) {
        if (a.scalar || !reads_input(a.spec, T)) continue;
        if (!reads_aligned(a.spec, T, shape) || sp.pos.at(c) > sp.pos.at(wop)) return false;
      }
    return true;
  }
  // (1): no entry after the writer reads T, and no entry before it that
  // reads T needs the writer's values (it could not then run first).
  bool other_reads_precede(int owner, const std::string& T, bool check_deps) const {
    for (size_t i = 0; i < sched.size(); ++i) {
      if ((int)i == owner || !entry_reads_input((int)i, T)) continue;
      if ((int)i > owner) return false;
      if (check_deps && depends_on((int)i, owner)) return false;
    }
    return true;
  }

  void prove_direct() {
    for (auto& kv : P.inplace) {
      const int slot = kv.first, tidx = kv.second;
      const Spec& out = P.outputs[slot];
      const std::string& T = P.inputs[tidx].buf;
      // the new value is returned once, through a whole contiguous view, and
      // the old one is not returned at all
      if (output_count[out.buf] != 1 || out.offset != 0 || !out.contiguous()) continue;
      if (output_bufs.count(T)) continue;
      const int owner = entry_writing(out.buf);
      if (owner < 0 || sched[owner].kind != 0) continue;
      const Entry& e = sched[owner];
      bool ok;
      if (op(e.op).cls == OC_POINTWISE && e.chain.empty() && e.side.empty()) {
        ok = plain_reads_in_step(e, T, out.shape) && other_reads_precede(owner, T, false);
      } else {
        int wop = -1;
        for (int c : e.side)
          if (op(c).out.buf == out.buf) wop = c;
        ok = wop >= 0 && tile_reads_in_step(e, wop, T, out.shape) && other_reads_precede(owner, T, true);
      }
      if (ok) direct[slot] = tidx;
    }
  }

  // Pass 3: fold a direct pointwise update into the contraction tile that
  // produces its only materialized operand.
  void pass3() {
    if (!O.fuse_updates || !O.fuse_epilogues) return;
    for (auto& kv : direct) {
      int slot = kv.first;
      const std::string& target = P.inputs[kv.second].buf;
      const std::string& ubuf = P.outputs[slot].buf;
      int uo = -1;
      for (size_t i = 0; i < sched.size(); ++i)
        if (sched[i].kind == 0 && sched[i].chain.empty() && sched[i].side.empty() && op(sched[i].op).out.buf == ubuf)
          uo = (int)i;
      if (uo < 0) continue;
      const Op& u = op(sched[uo].op);
      // the one operand produced by a contraction
      int mm_sched = -1;
      std::string mbuf;
      bool ok = true;
      for (auto& a : u.args) {
        if (a.scalar || is_input(a.spec.buf)) continue;
        if (inlined_bufs.count(a.spec.buf)) { ok = false; break; }
        int pj = prod(a.spec.buf);
        if (!is_contraction(pj)) { ok = false; break; }
        if (!mbuf.empty() && mbuf != a.spec.buf) { ok = false; break; }
        mbuf = a.spec.buf;
      }
      if (!ok || mbuf.empty()) continue;
      int mj = prod(mbuf);
      for (size_t i = 0; i < sched.size(); ++i)
        if (sched[i].kind == 0 && sched[i].op == mj) mm_sched = (int)i;
      if (mm_sched < 0) continue;
      Entry& me = sched[mm_sched];
      if (!me.chain.empty() || !me.side.empty()) continue;
      if (output_bufs.count(mbuf) || users[mbuf].size() != 1) continue;
      if (u.out.shape != op(mj).out.shape) continue;
      for (auto& a : u.args) {
        if (a.scalar) continue;
        if (a.spec.buf == mbuf && !identity_view(a.spec, op(mj).out.shape)) ok = false;
        if (a.spec.buf != mbuf && (a.spec.offset != 0 || !a.spec.contiguous())) ok = false;
      }
      // the tile must read nothing of the target
      for (auto& a : op(mj).args)
        if (!a.scalar && reads_input(a.spec, target)) ok = false;
      if (!ok) continue;
      // The fused tile takes the update's place in program order (after every
      // reader of the target), so ordering constraints stay acyclic.
      Entry fusedE = me;
      fusedE.chain.push_back(sched[uo].op);
      fusedE.update = true;
      skip.insert(sched[uo].op);
      sched[uo] = fusedE;
      sched.erase(sched.begin() + mm_sched);
    }
    for (size_t i = 0; i < sched.size(); ++i) sched[i].order = (int)i;
  }

  // ---------------------------------------------------------- bindings --
  // A stored value can be written straight into a caller's output buffer
  // when that output is exactly the value's own layout (same dtype and
  // element count, offset 0, contiguous): the value then needs no arena space
  // and no copy task.  Each value takes the first such output slot; every
  // other output of it gets a copy (add_copies_and_commits).  An in-place
  // output not proven direct never binds: its value goes to the arena and a
  // staged commit copies it into the target.
  static bool same_layout(const Spec& out, const Spec& value) {
    return out.dtype == value.dtype && out.offset == 0 && out.numel() == value.numel() && out.contiguous();
  }

  void bind_outputs() {
    std::set<std::string> stored;
    for (auto& e : sched)
      for (auto& w : written(e)) stored.insert(w);
    for (int s = 0; s < n_out; ++s) {
      const Spec& o2 = P.outputs[s];
      const bool staged = P.inplace.count(s) && !direct.count(s);
      if (staged || !stored.count(o2.buf) || bound.count(o2.buf)) continue;
      if (same_layout(o2, op(prod(o2.buf)).out)) bound[o2.buf] = s;
    }
    // Side-epilogue values are computed inside a contraction tile and have no
    // arena slot of their own; pass 2 only fuses a returned one when it can be
    // bound, so an unbound one here is a scheduler bug.
    for (auto& e : sched)
      for (int c : e.side) {
        const std::string& v = op(c).out.buf;
        if (output_bufs.count(v) && !aliased.count(v) && !bound.count(v))
          raise(TK_E_UNSUPPORTED, "internal: side epilogue without a direct output binding");
      }
  }

  // ---------------------------------------------------------- leveling --
  void add_copies_and_commits() {
    for (int s = 0; s < n_out; ++s) {
      const Spec& o2 = P.outputs[s];
      if (P.inplace.count(s) && !direct.count(s)) {
        Entry c;
        c.kind = 2;
        c.slot = s;
        c.writes_inputs = {P.inplace.at(s)};
        sched.push_back(c);
        continue;
      }
      auto b = bound.find(o2.buf);
      if (b != bound.end() && b->second == s) continue;
      Entry c;
      c.kind = 1;
      c.slot = s;
      sched.push_back(c);
    }
  }

  void collect_rw() {
    for (auto& e : sched) {
      e.reads_vals.clear();
      e.reads_inputs.clear();
      e.writes_vals.clear();
      if (e.kind == 0) {
        auto internal = internal_bufs(e);
        for (auto* a : entry_args(e)) {
          if (a->scalar || internal.count(a->spec.buf)) continue;
          root_values(a->spec, e.reads_vals);
          auto r = inputs_read(a->spec);
          e.reads_inputs.insert(r.begin(), r.end());
        }
        for (auto& w : written(e)) e.writes_vals.insert(w);
        e.writes_inputs.clear();
        for (auto& kv : direct)
          if (e.writes_vals.count(P.outputs[kv.first].buf)) e.writes_inputs.push_back(kv.second);
      } else {
        const Spec& o2 = P.outputs[e.slot];
        if (is_input(o2.buf))
          e.reads_inputs.insert(o2.buf);
        else
          e.reads_vals.push_back(o2.buf);
      }
    }
  }

  // Work items an entry puts into its stage (its first phase).
  uint64_t entry_items(const Entry& e) const {
    if (e.kind != 0) return ew_items(P.outputs[e.slot].numel());
    const Op& o2 = op(e.op);
    if (o2.cls == OC_POINTWISE) return ew_items(o2.out.numel());
    if (o2.cls == OC_REDUCE) {
      const RedChoice rc = choose_reduce(o2);
      if (rc.kind == T_RED_COLS) return (uint64_t)((rc.rows + 255) / 256) * rc.parts;
      return (uint64_t)rc.rows * rc.parts;
    }
    const GemmChoice g = choose_gemm(o2);
    return (uint64_t)g.tm * g.tn * std::max<uint32_t>(1, g.split);
  }

  // ------------------------------------------------ fused column sums --
  // A column reduction (sum or mean over dim 0) of a 2-D value V that is also
  // the B operand of a contraction (B(k, n) = V[k][n], whole and contiguous)
  // runs inside that contraction: its first tile row sums V's column block
  // over all of K (from the B fragments of its main loop, or by reading V
  // again after the tile; V is an input of the tile, unchanged in the stage)
  // and runs the reduction's finishing program per column.  Needed: an
  // unsplit matrix-core tile, the reduction's values read by no other entry,
  // and the reduction placed in the contraction's stage (its leveling
  // constraint below).  Typical case: the bias gradient of a layer summed from
  // the same gradient its weight-gradient product reads.  By default only
  // where the reduction's own items would give some workgroups of its stage
  // one more item than the rest have (otherwise they run on workgroups that
  // would idle anyway), and where K is not a multiple of 64 only up to 512
  // rows (the rows read again after the tile then cost less than a round of
  // items); colsum_fusion = 1 fuses wherever legal, -1 never.  Runs on a first leveling; the stages are
  // levelled again after.
  void fuse_column_sums() {
    if (!O.fuse_epilogues || !O.fast_epilogue || O.barrier_every_op || O.colsum_fusion < 0) return;
    const bool always = O.colsum_fusion > 0;
    const uint64_t G = (uint64_t)std::max(1, O.num_cus) * std::max(1, O.blocks_per_cu);
    std::map<int, uint64_t> stage_items;
    for (auto& e : sched) stage_items[e.level] += entry_items(e);
    std::map<std::string, int> readers;  // value -> entries reading it
    for (size_t i = 0; i < sched.size(); ++i)
      for (auto& v : sched[i].reads_vals) readers[v]++;
    for (size_t ri = 0; ri < sched.size(); ++ri) {
      const Entry& r = sched[ri];
      if (r.kind != 0 || op(r.op).cls != OC_REDUCE || colsum_host.count((int)ri)) continue;
      const Op& ro = op(r.op);
      const RedChoice rc = choose_reduce(ro);
      if (rc.kind != T_RED_COLS || ro.args.size() != 1 || ro.args[0].scalar) continue;
      const Spec& src = ro.args[0].spec;
      if (src.shape.size() != 2 || src.offset != 0 || !src.contiguous() || is_input(src.buf)) continue;
      if (inlined_bufs.count(src.buf) || src.dtype == DT_F32 || src.dtype == DT_I8) continue;
      if (rc.R != src.shape[0] || rc.rows != src.shape[1]) continue;
      bool used = false;  // another entry reads a value this reduction writes
      for (auto& w : r.writes_vals)
        if (readers.count(w)) used = true;
      if (used) continue;
      for (size_t xi = 0; xi < sched.size(); ++xi) {
        const Entry& x = sched[xi];
        if (x.kind != 0 || colsum_of.count((int)xi)) continue;
        const Op& mo = op(x.op);
        if (mo.cls != OC_MM) continue;
        const Spec& B = mo.B();
        if (B.buf != src.buf || B.shape != src.shape || B.offset != 0 || !B.contiguous()) continue;
        const GemmChoice g = choose_gemm(mo);
        if (g.kind != T_GEMM_MFMA || g.split > 1) continue;
        const uint64_t here = stage_items[r.level], own = entry_items(r);
        // K on whole 64-deep slices: the sums come out of the tile's main loop
        // (else the tile reads K rows again after the product)
        const bool in_loop = B.shape[0] % 64 == 0;
        if (!always && ((!in_loop && B.shape[0] > 512) || (here + G - 1) / G == (here - own + G - 1) / G)) continue;
        colsum_of[(int)xi] = (int)ri;
        colsum_host[(int)ri] = (int)xi;
        sched[ri].two_phase = false;
        break;
      }
    }
  }

  void level() {
    std::map<std::string, int> writer;
    for (size_t i = 0; i < sched.size(); ++i)
      for (auto& w : sched[i].writes_vals) writer[w] = (int)i;
    for (auto& e : sched) e.level = 0;
    for (int iter = 0; iter < 1000; ++iter) {
      bool changed = false;
      int prev_last = -1;
      for (size_t i = 0; i < sched.size(); ++i) {
        Entry& e = sched[i];
        int L = 0;
        for (auto& v : e.reads_vals) {
          auto it = writer.find(v);
          if (it == writer.end()) raise(TK_E_ARG, "internal: value '" + v + "' has no writer");
          if ((size_t)it->second != i) L = std::max(L, sched[it->second].avail() + 1);
        }
        for (int wi : e.writes_inputs) {
          const std::string& t = P.inputs[wi].buf;
          for (size_t r = 0; r < sched.size(); ++r)
            if (r != i && sched[r].reads_inputs.count(t)) L = std::max(L, sched[r].avail() + 1);
        }
        if (e.kind == 2) {  // staged commits also follow every other write of the step
          for (size_t r = 0; r < sched.size(); ++r)
            if (sched[r].kind == 0) L = std::max(L, sched[r].avail() + 1);
        }
        if (O.barrier_every_op && prev_last >= 0) L = std::max(L, prev_last + 1);
        // a column reduction run by a contraction shares its stage
        auto host = colsum_host.find((int)i);
        if (host != colsum_host.end()) L = std::max(L, sched[host->second].level);
        if (L != e.level) {
          e.level = L;
          changed = true;
        }
        prev_last = e.avail();
      }
      if (!changed) return;
    }
    raise(TK_E_ARG, "internal: leveling did not converge (cyclic dependencies)");
  }

  // ------------------------------------------------------------- arena --
  void plan_arena() {
    // Location of every stored value.
    for (auto& e : sched)
      for (auto& w : e.writes_vals) {
        Loc l;
        l.dtype = op(prod(w)).out.dtype;
        auto b = bound.find(w);
        if (b != bound.end()) {
          l.base = n_in + b->second;
          l.offset = 0;
        } else {
          l.base = ws_base;
        }
        loc[w] = l;
      }
    // Liveness in levels.
    std::map<std::string, int> wlevel, lastread;
    std::map<std::string, int> first_order;
    for (auto& e : sched)
      for (auto& w : e.writes_vals) {
        wlevel[w] = e.avail();
        lastread[w] = e.avail();
        first_order[w] = e.order;
      }
    for (auto& e : sched)
      for (auto& v : e.reads_vals) lastread[v] = std::max(lastread[v], e.avail());
    struct Block { std::string name; int start, last; uint64_t bytes; int order; int sched_idx; };
    std::vector<Block> blocks;
    for (auto& kv : loc) {
      if (kv.second.base != ws_base) continue;
      const Spec& pv = op(prod(kv.first)).out;
      uint64_t bytes = align_up(std::max<uint64_t>(1, pv.numel() * dtype_size(pv.dtype)), kAlign);
      blocks.push_back({kv.first, wlevel[kv.first], lastread[kv.first], bytes, first_order[kv.first], -1});
    }
    for (size_t i = 0; i < sched.size(); ++i)
      if (scratch_bytes.count((int)i))
        blocks.push_back({"#scratch" + std::to_string(i), sched[i].level, sched[i].avail(),
                          align_up(scratch_bytes[(int)i], kAlign), sched[i].order, (int)i});
    std::sort(blocks.begin(), blocks.end(), [](const Block& a, const Block& b) {
      return a.start != b.start ? a.start < b.start : a.order < b.order;
    });
    struct Live { uint64_t off, bytes; int last; };
    std::vector<Live> live;
    std::vector<std::pair<uint64_t, uint64_t>> freel;  // (offset, bytes)
    uint64_t top = 0;
    auto coalesce = [&]() {
      std::sort(freel.begin(), freel.end());
      std::vector<std::pair<uint64_t, uint64_t>> m;
      for (auto& f : freel) {
        if (!m.empty() && m.back().first + m.back().second == f.first)
          m.back().second += f.second;
        else
          m.push_back(f);
      }
      freel = m;
    };
    for (auto& b : blocks) {
      // release blocks whose last reader finished before this level
      std::vector<Live> keep;
      for (auto& l : live) {
        if (l.last < b.start)
          freel.push_back({l.off, l.bytes});
        else
          keep.push_back(l);
      }
      live = keep;
      coalesce();
      int best = -1;
      for (size_t i = 0; i < freel.size(); ++i)
        if (freel[i].second >= b.bytes && (best < 0 || freel[i].second < freel[best].second)) best = (int)i;
      uint64_t off;
      if (best >= 0) {
        off = freel[best].first;
        if (freel[best].second > b.bytes)
          freel[best] = {off + b.bytes, freel[best].second - b.bytes};
        else
          freel.erase(freel.begin() + best);
      } else {
        off = top;
        top += b.bytes;
      }
      live.push_back({off, b.bytes, b.last});
      if (b.sched_idx >= 0) {
        scratch_off[b.sched_idx] = kHeaderBytes + off;
      } else {
        arena_off[b.name] = off;
        Loc& l = loc[b.name];
        l.offset = (int64_t)((kHeaderBytes + off) / dtype_size(l.dtype));
      }
    }
    arena_bytes = top;
  }

  // ----------------------------------------------------- expressions --
  struct ExprCtx {
    std::vector<int64_t> space;  // task iteration shape (uncollapsed)
    std::vector<DView> vtab;     // views over `space` (uncollapsed, rank = space.size())
    std::map<std::string, int> slot_of;  // tile values held in slots
    std::set<std::string> expand;        // side values expanded into their reader
    const std::vector<int64_t>* flat = nullptr;  // read views over this shape flattened to 1-D
  };

  // A view as read over a flattened 1-D task space (see flattenable).
  static Spec flat_view(const Spec& s, const std::vector<int64_t>& shape) {
    Spec f = s;
    int64_t n = 1;
    for (auto d : shape) n *= d;
    f.shape = {n};
    f.strides = {(s.shape == shape && s.contiguous() && s.numel() != 1) ? 1 : 0};
    return f;
  }

  // A view of stored data over the task space: dims map[i] of the reading
  // op's space go to task dims (or -1: broadcast to coordinate 0).
  DView lift(const Spec& s, const std::vector<int>& map, const Loc& where, size_t rank) {
    DView v{};
    v.base = (uint16_t)where.base;
    v.dtype = s.dtype;
    v.offset = where.offset + s.offset;
    for (int d = 0; d < kMaxDims; ++d) v.stride[d] = 0;
    std::vector<int64_t> st(rank, 0);
    const size_t r = s.shape.size(), R = map.size();
    for (size_t j = 0; j < r; ++j) {
      if (s.shape[j] == 1) continue;
      int td = map[R - r + j];
      if (td < 0) continue;
      st[td] += s.strides[j];
    }
    // temporarily stash full-rank strides; collapsed later
    vstride_full.push_back(st);
    return v;
  }
  std::vector<std::vector<int64_t>> vstride_full;  // parallel to ExprCtx::vtab during building

  Loc storage_of(const std::string& buf) {
    if (is_input(buf)) {
      Loc l;
      l.base = input_idx[buf];
      l.offset = 0;
      l.dtype = P.inputs[input_idx[buf]].dtype;
      return l;
    }
    auto it = loc.find(buf);
    if (it == loc.end()) raise(TK_E_ARG, "internal: value '" + buf + "' has no storage");
    return it->second;
  }

  // Build the tree of an operand read through `s` by an op with iteration map `map`.
  Node operand_node(ExprCtx& cx, const Arg& a, const std::vector<int>& map) {
    Node n;
    if (a.scalar) {
      n.kind = Node::SCALAR;
      n.value = a.value;
      return n;
    }
    auto sl = cx.slot_of.find(a.spec.buf);
    if (sl != cx.slot_of.end()) {
      n.kind = Node::SLOT;
      n.slot = sl->second;
      return n;
    }
    if (cx.expand.count(a.spec.buf) || inlined_bufs.count(a.spec.buf)) {
      // identity view of the producer: its dims align with the view's dims
      std::vector<int> pm(a.spec.shape.size());
      const size_t r = a.spec.shape.size(), R = map.size();
      for (size_t j = 0; j < r; ++j) pm[j] = a.spec.shape[j] == 1 ? -1 : map[R - r + j];
      return op_node(cx, prod(a.spec.buf), pm);
    }
    n.kind = Node::LEAF;
    n.view = (int)cx.vtab.size();
    const Spec v = cx.flat ? flat_view(a.spec, *cx.flat) : a.spec;
    cx.vtab.push_back(lift(v, map, storage_of(a.spec.buf), cx.space.size()));
    return n;
  }

  Node op_node(ExprCtx& cx, int j, const std::vector<int>& map) {
    const Op& o2 = op(j);
    Node n;
    n.kind = Node::OP;
    n.op = j;
    for (auto& a : o2.args) n.kids.push_back(operand_node(cx, a, map));
    return n;
  }

  static bool simple(const Node& n) { return n.kind != Node::OP; }

  // Temporaries the accumulator machine needs for a node (Sethi-Ullman).
  int node_need(const Node& n) const {
    if (simple(n)) return 0;
    const Op& o2 = op(n.op);
    if (o2.opcode == "full" || n.kids.empty()) return 0;
    const bool binary = o2.opcode == "add" || o2.opcode == "sub" || o2.opcode == "mul" || o2.opcode == "div" ||
                        o2.opcode == "threshold_backward";
    const int nx = node_need(n.kids[0]);
    if (!binary) return nx;
    const Node &x = n.kids[0], &y = n.kids[1];
    const int ny = node_need(y);
    if (simple(y)) return nx;
    if (simple(x)) return ny;
    return ny > nx ? std::max(ny, 1 + nx) : std::max(nx, 1 + ny);
  }

  void emit_load(std::vector<DIns>& code, const Node& n) {
    DIns d{};
    d.op = VM_LOAD;
    d.rnd = RND_NONE;
    set_src(d, n);
    code.push_back(d);
  }
  static void set_src(DIns& d, const Node& n) {
    if (n.kind == Node::LEAF) {
      d.src = SRC_VIEW;
      d.arg = (uint16_t)n.view;
    } else if (n.kind == Node::SCALAR) {
      d.src = SRC_SCALAR;
      d.s = n.value;
    } else if (n.kind == Node::SLOT) {
      d.src = SRC_SLOT;
      d.arg = (uint16_t)n.slot;
    }
  }

  // Emit code leaving the node's value (rounded to its dtype) in the accumulator.
  // `busy`: slots holding values that must survive; temporaries take the
  // lowest free slots.
  static int lowest_free(uint32_t busy) {
    int k = 0;
    while (busy & (1u << k)) ++k;
    return k;
  }

  void emit(std::vector<DIns>& code, const Node& n, uint32_t busy) {
    if (simple(n)) {
      emit_load(code, n);
      return;
    }
    const Op& o2 = op(n.op);
    const std::string& c = o2.opcode;
    const uint8_t rnd = o2.out.dtype == DT_F32 ? RND_NONE : o2.out.dtype;
    DIns d{};
    d.rnd = rnd;
    auto unary = [&](uint8_t vop, float a) {
      emit(code, n.kids[0], busy);
      d.op = vop;
      d.a = a;
      d.src = SRC_NONE;
      code.push_back(d);
    };
    if (c == "full") {
      Node s;
      s.kind = Node::SCALAR;
      s.value = o2.attrs.count("value") ? o2.attrs.at("value") : (n.kids.empty() ? 0.0f : n.kids[0].value);
      emit_load(code, s);
      code.back().rnd = rnd;
      return;
    }
    if (c == "neg") return unary(VM_NEG, 0);
    if (c == "relu") return unary(VM_RELU, 0);
    if (c == "sqrt") return unary(VM_SQRT, 0);
    if (c == "cast") {
      emit(code, n.kids[0], busy);
      if (rnd != RND_NONE) {
        DIns r{};
        r.op = VM_SCALE;  // 1 * x is exact; the instruction carries the rounding
        r.a = 1.0f;
        r.rnd = rnd;
        code.push_back(r);
      }
      return;
    }
    if (c == "pow") {
      float e = n.kids.size() > 1 ? n.kids[1].value : o2.attr("exponent", 2.0f);
      if (e == 2.0f) return unary(VM_SQUARE, 0);
      return unary(VM_POW, e);
    }
    uint8_t vop = 0;
    float a = 0;
    if (c == "add") { vop = VM_ADD; a = o2.attr("alpha", 1.0f); }
    else if (c == "sub") { vop = VM_SUB; a = o2.attr("alpha", 1.0f); }
    else if (c == "mul") { vop = VM_MUL; }
    else if (c == "div") { vop = VM_DIV; }
    else if (c == "threshold_backward") { vop = VM_TB; a = o2.attr("threshold", 0.0f); }
    else raise(TK_E_UNSUPPORTED, "unsupported pointwise operation " + c);
    const Node &x = n.kids[0], &y = n.kids[1];
    d.op = vop;
    d.a = a;
    if (simple(y)) {
      emit(code, x, busy);
      set_src(d, y);
      d.rev = 0;
    } else if (simple(x)) {
      emit(code, y, busy);
      set_src(d, x);
      d.rev = 1;
    } else {
      // both operands are expressions: the one needing more temporaries
      // goes first, the other is computed while it waits in a slot
      const int t = lowest_free(busy);
      if (t >= kMaxSlots) raise(TK_E_UNSUPPORTED, "expression too deep for the tile program");
      const bool y_first = node_need(y) > node_need(x);
      emit(code, y_first ? y : x, busy);
      DIns sv{};
      sv.op = VM_SAVE;
      sv.arg = (uint16_t)t;
      sv.rnd = RND_NONE;
      code.push_back(sv);
      emit(code, y_first ? x : y, busy | (1u << t));
      d.src = SRC_SLOT;
      d.arg = (uint16_t)t;
      d.rev = y_first ? 0 : 1;
    }
    code.push_back(d);
  }

  void emit_store(std::vector<DIns>& code, ExprCtx& cx, const std::string& buf, const std::vector<int>& map) {
    const Spec& pv = op(prod(buf)).out;
    Spec s = cx.flat ? flat_view(pv, *cx.flat) : pv;  // contiguous view of the value itself
    DIns st{};
    st.op = VM_STORE;
    st.rnd = RND_NONE;
    st.arg = (uint16_t)cx.vtab.size();
    cx.vtab.push_back(lift(s, map, storage_of(buf), cx.space.size()));
    code.push_back(st);
  }

  // Collapse the task space and the views' strides; returns the collapsed dims.
  std::vector<int64_t> collapse(ExprCtx& cx, bool allow = true) {
    std::vector<int64_t> dims = cx.space;
    std::vector<std::vector<int64_t>> st = vstride_full;
    // drop size-1 dims
    std::vector<int64_t> d2;
    std::vector<std::vector<int64_t>> s2(st.size());
    for (size_t d = 0; d < dims.size(); ++d) {
      if (dims[d] == 1 && dims.size() > 1) continue;
      d2.push_back(dims[d]);
      for (size_t v = 0; v < st.size(); ++v) s2[v].push_back(st[v][d]);
    }
    dims = d2;
    st = s2;
    if (allow) {
      for (size_t d = 0; d + 1 < dims.size();) {
        bool ok = true;
        for (auto& s : st)
          if (s[d] != s[d + 1] * dims[d + 1]) ok = false;
        if (ok) {
          dims[d] *= dims[d + 1];
          dims.erase(dims.begin() + d + 1);
          for (auto& s : st) {
            s[d] = s[d + 1];
            s.erase(s.begin() + d + 1);
          }
        } else {
          ++d;
        }
      }
    }
    if (dims.empty()) {
      dims.push_back(1);
      for (auto& s : st) s.push_back(0);
    }
    if (dims.size() > (size_t)kMaxDims) raise(TK_E_UNSUPPORTED, "iteration space needs more than 4 dims after collapsing");
    for (size_t v = 0; v < cx.vtab.size(); ++v)
      for (size_t d = 0; d < dims.size(); ++d) cx.vtab[v].stride[d] = st[v][d];
    return dims;
  }

  uint32_t commit_views(ExprCtx& cx) {
    uint32_t first = (uint32_t)views.size();
    for (auto& v : cx.vtab) views.push_back(v);
    if (views.size() > 65000) raise(TK_E_UNSUPPORTED, "too many operand views");
    return first;
  }
  // Value-preserving clean-up of a program: an identity scale (1 * acc, no
  // rounding) goes, a reload of the slot just saved goes (the accumulator
  // still holds it), and a save nobody reads before the slot is overwritten
  // goes.  Every instruction the machine runs costs a dispatch.
  static void peephole(std::vector<DIns>& code) {
    for (bool changed = true; changed;) {
      changed = false;
      for (size_t i = 0; i < code.size(); ++i) {
        const DIns& d = code[i];
        if (d.op == VM_SCALE && d.a == 1.0f && d.rnd == RND_NONE && d.src == SRC_NONE) {
          code.erase(code.begin() + i);
          changed = true;
          break;
        }
        if (d.op == VM_SAVE && i + 1 < code.size()) {
          const DIns& n = code[i + 1];
          if (n.op == VM_LOAD && n.src == SRC_SLOT && n.arg == d.arg && n.rnd == RND_NONE) {
            code.erase(code.begin() + i + 1);
            changed = true;
            break;
          }
        }
      }
      if (changed) continue;
      // Slots whose value the accumulator still holds: a save makes its slot
      // equal to it, stores leave it alone, anything else changes it.
      uint32_t acc_eq = 0;
      for (size_t i = 0; i < code.size() && !changed; ++i) {
        DIns& d = code[i];
        const bool slot_equal = d.src == SRC_SLOT && d.arg < 32 && (acc_eq >> d.arg) & 1u;
        if (d.op == VM_LOAD && slot_equal && d.rnd == RND_NONE) {
          // reloading what the accumulator holds
          code.erase(code.begin() + i);
          changed = true;
        } else if (d.op == VM_LOAD && d.rnd == RND_NONE && (d.src == SRC_VIEW || d.src == SRC_SCALAR) &&
                   i + 1 < code.size()) {
          // load v ; op slot  ==>  op v with the operands' roles swapped,
          // when the slot's value is still in the accumulator
          DIns& n = code[i + 1];
          const bool binary = n.op == VM_ADD || n.op == VM_SUB || n.op == VM_MUL || n.op == VM_DIV || n.op == VM_TB;
          if (binary && n.src == SRC_SLOT && n.arg < 32 && ((acc_eq >> n.arg) & 1u)) {
            DIns r = n;
            r.src = d.src;
            r.arg = d.arg;
            r.s = d.s;
            r.rev = n.op == VM_MUL ? 0 : (n.rev ? 0 : 1);
            code[i] = r;
            code.erase(code.begin() + i + 1);
            changed = true;
          }
        }
        if (changed) break;
        if (d.op == VM_SAVE)
          acc_eq |= 1u << d.arg;
        else if (d.op != VM_STORE)
          acc_eq = 0;
      }
      if (changed) continue;
      for (size_t i = 0; i < code.size(); ++i) {
        const DIns& d = code[i];
        if (d.op == VM_SAVE) {
          bool read = false;
          for (size_t j = i + 1; j < code.size(); ++j) {
            if (code[j].src == SRC_SLOT && code[j].arg == d.arg && code[j].op != VM_SAVE && code[j].op != VM_STORE) {
              read = true;
              break;
            }
            if (code[j].op == VM_SAVE && code[j].arg == d.arg) break;
          }
          if (!read) {
            code.erase(code.begin() + i);
            changed = true;
            break;
          }
        }
      }
    }
  }

  // Whether a contraction tile's epilogue `code` (peepholed, view indices into
  // `vt`) over an m x n output, on tiles of `tile` x `tile`, can run as the
  // kernel's register program: a short straight-line program over 8-wide
  // column chunks, every view loaded once per chunk before the first
  // instruction runs.  Loads are hoisted, so a load may not follow a store
  // whose bytes it may read.  The unit-stride loaded views of a tile are
  // staged in the 48 KB of LDS above the fp32 tile: 16 bytes per 8-element
  // chunk and plane, two planes for fp32.
  static bool fast_epilogue_ok(const std::vector<DIns>& code, const std::vector<DView>& vt, int64_t m, int64_t n,
                               int tile) {
    if (n % 8 != 0 || m <= 0 || code.empty() || code.size() > (size_t)kFastIns) return false;
    int loads = 0;
    const int64_t plane = 16 * (int64_t)tile * tile / 8;
    const int64_t budget = (int64_t)kArenaBytes - (tile == 128 ? kFastStage128 : kFastStage64);
    int64_t staged = 0;
    auto range = [&](const DView& v, int64_t& lo, int64_t& hi) {
      const int64_t es = dtype_size(v.dtype);
      int64_t a = v.offset, b = v.offset;
      const int64_t ext[2] = {m - 1, n - 1};
      for (int d = 0; d < 2; ++d) {
        const int64_t step = v.stride[d] * ext[d];
        if (step < 0) a += step; else b += step;
      }
      lo = a * es;
      hi = (b + 1) * es;
    };
    for (size_t i = 0; i < code.size(); ++i) {
      const DIns& d = code[i];
      switch (d.op) {
        case VM_LOAD: case VM_ADD: case VM_SUB: case VM_MUL: case VM_DIV: case VM_NEG: case VM_RELU:
        case VM_SQUARE: case VM_TB: case VM_STORE: case VM_SCALE: case VM_ZERO: break;
        default: return false;
      }
      if (d.src == SRC_SLOT) return false;
      const bool is_store = d.op == VM_STORE;
      if (d.src != SRC_VIEW && !is_store) continue;
      if (d.arg >= vt.size()) return false;
      const DView& v = vt[d.arg];
      if (v.dtype == DT_I8) return false;
      for (int k = 2; k < kMaxDims; ++k)
        if (v.stride[k] != 0) return false;
      const int64_t s1 = v.stride[1], epc = v.dtype == DT_F32 ? 4 : 8;
      if (is_store ? s1 != 1 : (s1 != 1 && s1 != 0)) return false;
      if (s1 == 1 && (v.offset % epc != 0 || v.stride[0] % epc != 0)) return false;
      if (is_store) continue;
      if (++loads > kFastLoads) return false;
      if (s1 == 1 && (staged += (v.dtype == DT_F32 ? 2 : 1) * plane) > budget) return false;
      int64_t lo, hi;
      range(v, lo, hi);
      for (size_t j = 0; j < i; ++j) {
        if (code[j].op != VM_STORE) continue;
        const DView& w = vt[code[j].arg];
        if (w.base != v.base) continue;
        int64_t wlo, whi;
        range(w, wlo, whi);
        if (lo < whi && wlo < hi) return false;
      }
    }
    return true;
  }

  // The register epilogue's records (plan.h): for each committed
  // instruction, the instruction (with its staged chunks' arena offset) and
  // its view resolved to base, dtype, offset and strides.  Staged offsets are
  // assigned in program order, as the kernel copies the views.
  uint32_t fast_records(uint32_t code_first, uint32_t len, int tile) {
    const uint32_t first = (uint32_t)ins.size();
    const uint32_t plane = 16u * (uint32_t)tile * (uint32_t)tile / 8u;
    uint32_t staged = tile == 128 ? kFastStage128 : kFastStage64;
    for (uint32_t i = 0; i < len; ++i) {
      DIns a = ins.at(code_first + i), b{};
      a.pad = kFastNotStaged;
      if (a.src == SRC_VIEW || a.op == VM_STORE) {
        const DView& v = views.at(a.arg);
        b.rnd = v.dtype;
        b.rev = v.stride[1] == 1 ? 1 : 0;
        b.arg = v.base;
        const int32_t off = (int32_t)v.offset, s0 = (int32_t)v.stride[0];
        std::memcpy(&b.a, &off, 4);
        std::memcpy(&b.s, &s0, 4);
        if (a.op != VM_STORE && v.stride[1] == 1) {
          a.pad = (uint16_t)(staged / 16);
          staged += (v.dtype == DT_F32 ? 2u : 1u) * plane;
          if (staged > kArenaBytes) raise(TK_E_ARG, "internal: register epilogue operands exceed the arena");
        }
      }
      ins.push_back(a);
      ins.push_back(b);
    }
    return first;
  }

  uint32_t commit_code(std::vector<DIns>& code, uint32_t view_base) {
    peephole(code);
    uint32_t first = (uint32_t)ins.size();
    for (auto d : code) {
      if (d.src == SRC_VIEW || d.op == VM_STORE) d.arg = (uint16_t)(d.arg + view_base);
      ins.push_back(d);
    }
    return first;
  }

  // --------------------------------------------------------- planning --
  struct GemmChoice { uint8_t kind; uint8_t tile; uint32_t split, kchunk, tm, tn; };

  GemmChoice choose_gemm(const Op& mm) const {
    const Spec &A = mm.A(), &B = mm.B();
    const int64_t m = A.shape[0], k = A.shape[1], n = mm.out.shape[1];
    GemmChoice g{};
    if (mm.cls == OC_MM_Q8) {
      // slabs of kGemvRows activation rows share each weight chunk they load
      g.kind = T_GEMV_Q8;
      g.tm = (uint32_t)((m + kGemvRows - 1) / kGemvRows);
      g.tn = (uint32_t)((n + 15) / 16);
      g.split = 1;
      return g;
    }
    const bool mfma_dtype = A.dtype == B.dtype && (A.dtype == DT_BF16 || A.dtype == DT_F16);
    if (!mfma_dtype || m <= 4 || k <= 8 || n <= 4) {
      g.kind = T_GEMM_SIMT;
      g.tile = 0;
      g.tm = (uint32_t)((m + 63) / 64);
      g.tn = (uint32_t)((n + 63) / 64);
      g.split = 1;
      g.kchunk = (uint32_t)k;
      return g;
    }
    g.kind = T_GEMM_MFMA;
    const double G = (double)O.num_cus * std::max(1, O.blocks_per_cu);
    double best = 1e300;
    const int tiles[2][2] = {{128, 128}, {64, 64}};
    const double eff[2] = {1.0, 0.55};
    for (int t = 0; t < 2; ++t) {
      if (O.gemm_tile > 0 && t != O.gemm_tile - 1) continue;
      const int bm = tiles[t][0], bn = tiles[t][1];
      const int64_t tm = (m + bm - 1) / bm, tn = (n + bn - 1) / bn;
      for (int S : {1, 2, 4, 8}) {
        if (O.gemm_split_k > 0 && S != O.gemm_split_k) continue;
        int64_t kc = ((k + S - 1) / S + 63) / 64 * 64;
        int64_t Se = (k + kc - 1) / kc;
        if (Se != S) continue;
        if (S > 1 && kc < 256 && O.gemm_split_k == 0) continue;
        double items = (double)(tm * tn * Se);
        double waves = std::ceil(items / G);
        double t_us = waves * (2.0 * bm * bn * kc) / (9.8e12 * eff[t]) * 1e6;
        if (Se > 1) t_us += (double)m * n * Se * 8.0 / 6e12 * 1e6 + 3.0;
        if (t_us < best - 1e-9) {
          best = t_us;
          g.tile = (uint8_t)t;
          g.split = (uint32_t)Se;
          g.kchunk = (uint32_t)kc;
          g.tm = (uint32_t)tm;
          g.tn = (uint32_t)tn;
        }
      }
    }
    if (best >= 1e300) raise(TK_E_UNSUPPORTED, "no GEMM tiling for the requested split");
    return g;
  }

  // Reduction geometry.
  struct RedChoice {
    uint8_t kind;              // T_RED_ROWS / T_RED_COLS
    std::vector<int> perm;     // iteration order of the source dims
    int64_t rows, R;           // kept size, reduced size
    uint32_t parts, kchunk;    // parts per output (rows) / row parts (cols)
    bool colform;
  };

  RedChoice choose_reduce(const Op& r) const {
    const Spec& x = r.args[0].spec;
    const int rank = (int)x.shape.size();
    std::vector<bool> red(rank, false);
    if (r.dims_all) {
      for (int d = 0; d < rank; ++d) red[d] = true;
    } else {
      for (auto d : r.dims) red[((d % rank) + rank) % rank] = true;
    }
    RedChoice c{};
    int64_t kept = 1, rr = 1;
    for (int d = 0; d < rank; ++d) (red[d] ? rr : kept) *= x.shape[d];
    c.rows = kept;
    c.R = rr;
    // leading-dims reduction -> column form
    int first_kept = rank;
    for (int d = 0; d < rank; ++d)
      if (!red[d]) { first_kept = d; break; }
    bool prefix = true;
    for (int d = first_kept; d < rank; ++d)
      if (red[d]) prefix = false;
    c.colform = prefix && first_kept > 0 && first_kept < rank;
    if (c.colform) {
      c.kind = T_RED_COLS;
      for (int d = 0; d < rank; ++d) c.perm.push_back(d);
      // 32 rows per part: a work item is at most two machine batches (8 row
      // lanes x 2 rows per batch for 8-wide chunks), so parts run in parallel
      // across workgroups instead of in sequence within one
      // (up to 64 rows stay one part: a combine stage would cost more).  A
      // source read straight from memory (an input or a materialised value,
      // summed without batches) stays one part up to 256 rows: 32 loads per
      // thread cost less than the combine stage and its barrier.
      const Arg& src = r.args[0];
      const int sp = src.scalar ? -2 : prod(src.spec.buf);
      const bool direct = !src.scalar && src.spec.dtype != DT_I8 && (sp == -1 || (sp >= 0 && !inlined.count(sp)));
      // A direct source contiguous along its kept dim with outputs in 8-wide
      // chunks takes the kernel's 32-row-lane form (64 columns per item, up
      // to 32 rows per lane): one part from 513 to 1024 rows, no combine
      // stage.  (Measured on MI355X: at 512 rows, 16 parts of 32 rows and a
      // combine in the next stage finish sooner than 16 rows per lane.)
      const bool lanes32 = direct && O.fast_epilogue && kept % 8 == 0 && !src.spec.strides.empty() &&
                           src.spec.strides.back() == 1;
      int64_t parts = (rr <= 64 || (direct && rr <= 256) || (lanes32 && rr > 512 && rr <= 1024))
                          ? 1
                          : std::min<int64_t>(64, (rr + 31) / 32);
      int64_t kc = (rr + parts - 1) / parts;
      parts = (rr + kc - 1) / std::max<int64_t>(1, kc);
      c.parts = (uint32_t)std::max<int64_t>(1, parts);
      c.kchunk = (uint32_t)std::max<int64_t>(1, kc);
    } else {
      c.kind = T_RED_ROWS;
      for (int d = 0; d < rank; ++d)
        if (!red[d]) c.perm.push_back(d);
      for (int d = 0; d < rank; ++d)
        if (red[d]) c.perm.push_back(d);
      int64_t parts = std::min<int64_t>(256, std::max<int64_t>(1, (rr + 4095) / 4096));
      int64_t kc = ((rr + parts - 1) / parts + 7) / 8 * 8;
      parts = rr == 0 ? 1 : (rr + kc - 1) / kc;
      c.parts = (uint32_t)std::max<int64_t>(1, parts);
      c.kchunk = (uint32_t)std::max<int64_t>(8, kc);
    }
    return c;
  }

  bool two_phase_of(const Entry& e) const {
    if (e.kind != 0) return false;
    const Op& o2 = op(e.op);
    if (o2.cls == OC_MM || o2.cls == OC_MM_Q8) return choose_gemm(o2).split > 1;
    if (o2.cls == OC_REDUCE) return choose_reduce(o2).parts > 1;
    return false;
  }

  void size_scratch() {
    for (size_t i = 0; i < sched.size(); ++i) {
      const Entry& e = sched[i];
      if (!e.two_phase) continue;
      const Op& o2 = op(e.op);
      if (o2.cls == OC_REDUCE) {
        auto rc = choose_reduce(o2);
        scratch_bytes[(int)i] = (uint64_t)rc.rows * rc.parts * 4;
      } else {
        auto g = choose_gemm(o2);
        scratch_bytes[(int)i] = (uint64_t)g.split * o2.out.numel() * 4;
      }
    }
  }

  // ------------------------------------------------------ task emission --
  void put(int level, DTask t, const std::string& desc) {
    if ((int)stage_tasks.size() <= level) {
      stage_tasks.resize(level + 1);
      stage_desc.resize(level + 1);
    }
    stage_tasks[level].push_back(t);
    stage_desc[level].push_back(desc);
  }

  static DTask blank(uint8_t kind) {
    DTask t;
    std::memset(&t, 0, sizeof(t));
    t.kind = kind;
    t.width = 1;
    t.ndim = 1;
    for (int d = 0; d < kMaxDims; ++d) t.dims[d] = 1;
    return t;
  }

  // Constants for dividing 32-bit unsigned values by dims[d] (d >= 1) with a
  // multiply-high and shifts, exact for every dividend below 2^32
  // (Granlund and Montgomery, "Division by invariant integers using
  // multiplication", 1994, figure 4.1).
  static void set_divisors(DTask& t) {
    for (int d = 0; d < kMaxDims; ++d) {
      t.dmul[d] = 0;
      t.dsh[d] = 0;
    }
    for (int d = 1; d < (int)t.ndim && d < kMaxDims; ++d) {
      const uint64_t dv = t.dims[d] ? t.dims[d] : 1;
      uint32_t l = 0;
      while ((1ull << l) < dv) ++l;
      t.dmul[d] = (uint32_t)(((1ull << 32) * ((1ull << l) - dv)) / dv + 1);
      t.dsh[d] = (uint8_t)l;
    }
  }

  // Elementwise work item: 4096 elements (16 per thread).
  static uint32_t ew_items(int64_t numel) { return (uint32_t)std::max<int64_t>(1, (numel + 4095) / 4096); }

  void emit_pointwise(const Entry& e) {
    const Op& o2 = op(e.op);
    ExprCtx cx;
    vstride_full.clear();
    cx.space = o2.out.shape;
    std::vector<int> map(cx.space.size());
    for (size_t d = 0; d < map.size(); ++d) map[d] = (int)d;
    Node root = op_node(cx, e.op, map);
    std::vector<DIns> code;
    emit(code, root, 0u);
    emit_store(code, cx, o2.out.buf, map);
    auto dims = collapse(cx);
    DTask t = blank(T_EW);
    t.ndim = (uint8_t)dims.size();
    for (size_t d = 0; d < dims.size(); ++d) t.dims[d] = (uint32_t)dims[d];
    t.width = (dims.back() % 8 == 0) ? 8 : 1;
    uint32_t vb = commit_views(cx);
    t.expr_first = commit_code(code, vb);
    t.expr_len = (uint32_t)code.size();
    t.n_items = o2.out.numel() == 0 ? 0 : ew_items(o2.out.numel());
    put(e.level, t, o2.name + " (" + o2.opcode + ")");
  }

  // Output copy or staged commit: read the value through the output view,
  // convert to the output dtype, write the destination contiguously.
  void emit_copy(const Entry& e) {
    const Spec& o2 = P.outputs[e.slot];
    ExprCtx cx;
    vstride_full.clear();
    cx.space = o2.shape;
    std::vector<int> map(cx.space.size());
    for (size_t d = 0; d < map.size(); ++d) map[d] = (int)d;
    std::vector<DIns> code;
    DIns ld{};
    ld.op = VM_LOAD;
    ld.src = SRC_VIEW;
    ld.rnd = RND_NONE;
    ld.arg = (uint16_t)cx.vtab.size();
    Spec src = o2;
    Loc sl = storage_of(o2.buf);
    src.dtype = sl.dtype;
    cx.vtab.push_back(lift(src, map, sl, cx.space.size()));
    code.push_back(ld);
    Spec dst = o2;
    dst.strides.clear();
    int64_t acc = 1;
    dst.strides.resize(o2.shape.size());
    for (size_t i = o2.shape.size(); i-- > 0;) {
      dst.strides[i] = acc;
      acc *= o2.shape[i];
    }
    dst.offset = 0;
    Loc dl;
    dl.base = n_in + e.slot;
    dl.offset = 0;
    dl.dtype = o2.dtype;
    DIns st{};
    st.op = VM_STORE;
    st.rnd = RND_NONE;
    st.arg = (uint16_t)cx.vtab.size();
    cx.vtab.push_back(lift(dst, map, dl, cx.space.size()));
    code.push_back(st);
    auto dims = collapse(cx);
    DTask t = blank(T_EW);
    t.ndim = (uint8_t)dims.size();
    for (size_t d = 0; d < dims.size(); ++d) t.dims[d] = (uint32_t)dims[d];
    t.width = (dims.back() % 8 == 0) ? 8 : 1;
    uint32_t vb = commit_views(cx);
    t.expr_first = commit_code(code, vb);
    t.expr_len = (uint32_t)code.size();
    t.n_items = o2.numel() == 0 ? 0 : ew_items(o2.numel());
    put(e.level, t, std::string(e.kind == 2 ? "commit" : "copy") + " out[" + std::to_string(e.slot) + "] <- " + o2.buf);
  }

  // Epilogue of a contraction tile, over the [m, n] output space.
  void build_epilogue(const Entry& e, ExprCtx& cx, std::vector<DIns>& code) {
    const Op& mm = op(e.op);
    std::vector<int> map = {0, 1};
    // root = alpha*acc + beta*bias (addmm forms), rounded to the root dtype
    const uint8_t rrnd = mm.out.dtype == DT_F32 ? RND_NONE : mm.out.dtype;
    if (mm.has_bias()) {
      float alpha = mm.attr("alpha", 1.0f), beta = mm.attr("beta", 1.0f);
      if (alpha == 0.0f && beta == 0.0f) {
        DIns z{};
        z.op = VM_ZERO;
        z.rnd = rrnd;
        code.push_back(z);
      } else if (beta == 0.0f) {
        DIns s{};
        s.op = VM_SCALE;
        s.a = alpha;
        s.rnd = rrnd;
        code.push_back(s);
      } else if (alpha == 0.0f) {
        Node b = operand_node(cx, mm.args[0], map);
        emit(code, b, 1u);
        DIns s{};
        s.op = VM_SCALE;
        s.a = beta;
        s.rnd = rrnd;
        code.push_back(s);
      } else {
        DIns s{};
        s.op = VM_SCALE;
        s.a = alpha;
        s.rnd = RND_NONE;
        code.push_back(s);
        Node b = operand_node(cx, mm.args[0], map);
        if (simple(b)) {
          DIns ad{};
          ad.op = VM_ADD;
          ad.a = beta;
          ad.rnd = rrnd;
          set_src(ad, b);
          code.push_back(ad);
        } else {
          DIns sv{};
          sv.op = VM_SAVE;
          sv.arg = 0;
          sv.rnd = RND_NONE;
          code.push_back(sv);
          emit(code, b, 1u);  // bias expression
          DIns ad{};
          ad.op = VM_ADD;  // acc(bias) ; slot0 + beta*acc
          ad.a = beta;
          ad.rev = 1;
          ad.src = SRC_SLOT;
          ad.arg = 0;
          ad.rnd = rrnd;
          code.push_back(ad);
        }
      }
    } else if (rrnd != RND_NONE) {
      DIns s{};
      s.op = VM_SCALE;
      s.a = 1.0f;
      s.rnd = rrnd;
      code.push_back(s);
    }
    if (!e.side.empty()) {
      emit_side_program(e, cx, code, map);
      return;
    }
    std::string cur = mm.out.buf;
    for (int c : e.chain) {
      DIns sv{};
      sv.op = VM_SAVE;
      sv.arg = 0;
      sv.rnd = RND_NONE;
      code.push_back(sv);
      cx.slot_of.clear();
      cx.slot_of[cur] = 0;
      Node n = op_node(cx, c, map);
      emit(code, n, 1u);
      cur = op(c).out.buf;
    }
    cx.slot_of.clear();
    emit_store(code, cx, cur, map);
  }

  // The root value is in the accumulator: hold it if side ops read it, store
  // it unless discarded, then evaluate the side ops as plan_side laid out.
  void emit_side_program(const Entry& e, ExprCtx& cx, std::vector<DIns>& code, const std::vector<int>& map) {
    const std::string& root = op(e.op).out.buf;
    const SidePlan sp = plan_side(e, inlined_bufs);
    if (!sp.ok) raise(TK_E_UNSUPPORTED, "internal: side program of " + op(e.op).name + " exceeds the slot budget");
    cx.expand = sp.expanded;
    auto save = [&](int slot) {
      DIns sv{};
      sv.op = VM_SAVE;
      sv.arg = (uint16_t)slot;
      sv.rnd = RND_NONE;
      code.push_back(sv);
    };
    if (sp.slot.count(root)) {
      save(0);
      cx.slot_of[root] = 0;
    }
    if (!e.discard_root) emit_store(code, cx, root, map);
    for (size_t i = 0; i < sp.evals.size(); ++i) {
      const int c = sp.evals[i];
      Node n = op_node(cx, c, map);
      emit(code, n, sp.busy[i]);
      const std::string& ob = op(c).out.buf;
      if (side_stored(e, c)) emit_store(code, cx, ob, map);
      auto it = sp.slot.find(ob);
      if (it != sp.slot.end()) {
        save(it->second);
        cx.slot_of[ob] = it->second;
      }
    }
  }

  DView operand_view(const Spec& s, int d0, int d1) {
    // A rank-two operand: stride[0] along its first index, stride[1] along its second.
    Loc l = storage_of(s.buf);
    DView v{};
    v.base = (uint16_t)l.base;
    v.dtype = s.dtype;
    v.offset = l.offset + s.offset;
    v.stride[0] = s.strides[d0];
    v.stride[1] = s.strides[d1];
    return v;
  }

  void emit_contraction(size_t si) {
    const Entry& e = sched[si];
    const Op& mm = op(e.op);
    const Spec &A = mm.A(), &B = mm.B();
    const int64_t m = A.shape[0], k = A.shape[1], n = mm.out.shape[1];
    GemmChoice g = choose_gemm(mm);
    ExprCtx cx;
    vstride_full.clear();
    cx.space = {m, n};
    std::vector<DIns> code;
    build_epilogue(e, cx, code);
    // no collapsing: epilogues address (row, col)
    for (size_t v = 0; v < cx.vtab.size(); ++v) {
      cx.vtab[v].stride[0] = vstride_full[v][0];
      cx.vtab[v].stride[1] = vstride_full[v][1];
    }
    DTask t = blank(g.kind);
    t.ndim = 2;
    t.dims[0] = (uint32_t)m;
    t.dims[1] = (uint32_t)n;
    t.m = (uint32_t)m;
    t.n = (uint32_t)n;
    t.k = (uint32_t)k;
    t.tile = g.tile;
    t.split = g.split;
    t.kchunk = g.kchunk;
    t.tiles_m = g.tm;
    t.tiles_n = g.tn;
    t.width = (n % 8 == 0) ? 8 : 1;
    // Tile order: the kernel gives each XCD a contiguous run of tiles/8 tiles
    // (when the count divides by 8); in group-major order (group_m tile rows
    // at a time, column by column) such a run is a group_m x (run/group_m)
    // block, whose operand panels the XCD's L2 shares.  Choose the block that
    // touches the fewest panels.
    t.group_m = 1;
    {
      const uint64_t tiles = (uint64_t)g.tm * g.tn;
      const uint64_t run = tiles % 8 == 0 ? tiles / 8 : tiles;
      uint64_t best = run + 1;
      for (uint64_t d = 1; d <= g.tm; ++d) {
        if (g.tm % d || run % d || run / d > g.tn) continue;
        if (d + run / d < best) {
          best = d + run / d;
          t.group_m = (uint32_t)d;
        }
      }
    }
    // operand views go first in this task's view block
    std::vector<DView> ops;
    if (g.kind == T_GEMV_Q8) {
      ops.push_back(operand_view(A, 0, 1));       // x over (row, k)
      ops.push_back(operand_view(B, 0, 1));       // q over (n, k)
      ops.push_back(operand_view(mm.S(), 0, 1));  // s over (n, block)
      if (mm.attrs.count("xq") && mm.attrs.at("xq") != 0.0f) t.flags |= F_XQ;
    } else {
      ops.push_back(operand_view(A, 0, 1));  // A over (m, k)
      ops.push_back(operand_view(B, 0, 1));  // B over (k, n)
    }
    uint32_t vbase = (uint32_t)views.size();
    for (auto& v : ops) views.push_back(v);
    t.va = (uint16_t)vbase;
    t.vb = (uint16_t)(vbase + 1);
    t.vs = (uint16_t)(vbase + (ops.size() > 2 ? 2 : 1));
    uint32_t vb = commit_views(cx);
    uint32_t code_first = commit_code(code, vb);
    const int fast_tile = g.kind == T_GEMM_MFMA && g.tile == 0 ? 128 : 64;
    if ((g.kind == T_GEMM_MFMA || g.kind == T_GEMM_SIMT) && g.split <= 1 && O.fast_epilogue &&
        fast_epilogue_ok(code, cx.vtab, m, n, fast_tile)) {
      t.flags |= F_FASTEPI;
      t.fin_first = fast_records(code_first, (uint32_t)code.size(), fast_tile);
      t.fin_len = 2 * (uint32_t)code.size();
    }
    std::string desc = mm.name + " (" + mm.opcode + " " + std::to_string(m) + "x" + std::to_string(k) + "x" +
                       std::to_string(n) + ")";
    if (t.flags & F_FASTEPI) desc += " [register epilogue]";
    auto cs = colsum_of.find((int)si);
    if (cs != colsum_of.end()) {
      // the fused column reduction's finishing program, over its n outputs
      const Entry& re = sched[cs->second];
      const Op& ro = op(re.op);
      t.flags |= F_BSUM;
      t.bs_first = reduction_finish(re, choose_reduce(ro));
      t.bs_len = last_finish_len;
      std::string rd = ro.name + " (" + ro.opcode + " " + std::to_string(n) + " outputs over " + std::to_string(k) + ")";
      if (!re.side.empty()) {
        rd += " +side";
        for (int c : re.side) rd += " " + op(c).name;
        if (re.discard_root) rd += " (root discarded)";
      }
      desc += " +column sums of B: " + rd;
    }
    if (t.flags & F_XQ) desc += " [activations quantised to Q8_0]";
    if (!e.chain.empty()) {
      desc += e.update ? " +update" : " +epilogue";
      for (int c : e.chain) desc += " " + op(c).name;
    }
    if (!e.side.empty()) {
      desc += " +side";
      for (int c : e.side) desc += " " + op(c).name;
      if (e.discard_root) desc += " (root discarded)";
    }
    if (g.split > 1) {
      DTask p1 = t;
      p1.flags |= F_PARTIAL;
      p1.scratch = scratch_off.at((int)si);
      p1.n_items = g.tm * g.tn * g.split;
      p1.expr_first = 0;
      p1.expr_len = 0;
      put(e.level, p1, desc + " [split-K " + std::to_string(g.split) + " partials]");
      DTask p2 = blank(T_GEMM_REDUCE);
      p2.ndim = 2;
      p2.dims[0] = (uint32_t)m;
      p2.dims[1] = (uint32_t)n;
      p2.m = (uint32_t)m;
      p2.n = (uint32_t)n;
      p2.split = g.split;
      p2.scratch = p1.scratch;
      p2.width = (n % 8 == 0) ? 8 : 1;
      p2.expr_first = code_first;
      p2.expr_len = (uint32_t)code.size();
      p2.n_items = ew_items(m * n);
      put(e.level + 1, p2, desc + " [split-K reduce + epilogue]");
    } else {
      t.expr_first = code_first;
      t.expr_len = (uint32_t)code.size();
      t.n_items = (m * n == 0) ? 0 : g.tm * g.tn;
      put(e.level, t, desc);
    }
    if (g.kind == T_GEMM_MFMA) st.matrix_core_ops++;
  }

  // The finishing program of a reduction over its `rows` outputs (1-D): the
  // mean's division, the rounding to the output dtype, then the side program
  // (or the store of the root).  Returns its first instruction; its length is
  // left in last_finish_len.
  uint32_t last_finish_len = 0;
  uint32_t reduction_finish(const Entry& e, const RedChoice& rc) {
    const Op& r = op(e.op);
    ExprCtx fx;
    vstride_full.clear();
    fx.space = {rc.rows};
    std::vector<DIns> fin;
    if (r.opcode == "mean") {
      DIns dv{};
      dv.op = VM_DIV;
      dv.src = SRC_SCALAR;
      dv.s = (float)rc.R;
      dv.rnd = RND_NONE;
      fin.push_back(dv);
    }
    if (r.out.dtype != DT_F32) {
      DIns s{};
      s.op = VM_SCALE;
      s.a = 1.0f;
      s.rnd = r.out.dtype;
      fin.push_back(s);
    }
    if (!e.side.empty()) {
      // side ops over the outputs, addressed as one flat index
      if (r.out.shape.size() != 1) fx.flat = &r.out.shape;
      emit_side_program(e, fx, fin, {0});
      for (size_t v = 0; v < fx.vtab.size(); ++v) fx.vtab[v].stride[0] = vstride_full[v][0];
    } else {
      Spec flat = r.out;
      flat.shape = {rc.rows};
      flat.strides = {1};
      DIns stv{};
      stv.op = VM_STORE;
      stv.rnd = RND_NONE;
      stv.arg = (uint16_t)fx.vtab.size();
      std::vector<int> m1 = {0};
      fx.vtab.push_back(lift(flat, m1, storage_of(r.out.buf), 1));
      fin.push_back(stv);
      fx.vtab.back().stride[0] = vstride_full.back()[0];
    }
    uint32_t fvb = commit_views(fx);
    const uint32_t first = commit_code(fin, fvb);  // (the peephole may shorten fin)
    last_finish_len = (uint32_t)fin.size();
    return first;
  }

  void emit_reduction(size_t si) {
    const Entry& e = sched[si];
    const Op& r = op(e.op);
    RedChoice rc = choose_reduce(r);
    const Spec& x = r.args[0].spec;
    // source expression over the permuted source space
    ExprCtx cx;
    vstride_full.clear();
    for (int d : rc.perm) cx.space.push_back(x.shape[d]);
    // map from the source op's own dims to the permuted task dims
    std::vector<int> map(x.shape.size());
    for (size_t i = 0; i < rc.perm.size(); ++i) map[rc.perm[i]] = (int)i;
    Node src = operand_node(cx, r.args[0], map);
    std::vector<DIns> code;
    emit(code, src, 0u);
    // collapse kept and reduced parts separately
    std::vector<int64_t> dims;
    {
      // Collapse within the kept group and within the reduced group only.
      std::vector<int64_t> full = cx.space;
      // number of leading (permuted) dims in the first group: the reduced
      // prefix for the column form, the kept dims for the row form
      const int rank = (int)x.shape.size();
      std::vector<bool> red(rank, r.dims_all);
      for (auto dd : r.dims) red[((dd % rank) + rank) % rank] = true;
      int split_at = 0;
      for (int d = 0; d < rank; ++d)
        if (red[d] == rc.colform) split_at++;
      auto group = [&](int lo, int hi, std::vector<int64_t>& gd, std::vector<std::vector<int64_t>>& gs) {
        for (int d = lo; d < hi; ++d) {
          if (full[d] == 1) continue;
          if (!gd.empty()) {
            bool ok = true;
            for (size_t v = 0; v < vstride_full.size(); ++v)
              if (gs[v].back() != vstride_full[v][d] * full[d]) ok = false;
            if (ok) {
              gd.back() *= full[d];
              for (size_t v = 0; v < vstride_full.size(); ++v) gs[v].back() = vstride_full[v][d];
              continue;
            }
          }
          gd.push_back(full[d]);
          for (size_t v = 0; v < vstride_full.size(); ++v) gs[v].push_back(vstride_full[v][d]);
        }
        if (gd.empty()) {
          gd.push_back(1);
          for (size_t v = 0; v < vstride_full.size(); ++v) gs[v].push_back(0);
        }
      };
      std::vector<int64_t> g1, g2;
      std::vector<std::vector<int64_t>> s1(vstride_full.size()), s2(vstride_full.size());
      group(0, split_at, g1, s1);
      group(split_at, (int)full.size(), g2, s2);
      if (g1.size() + g2.size() > (size_t)kMaxDims) raise(TK_E_UNSUPPORTED, "reduction needs more than 4 iteration dims");
      dims = g1;
      dims.insert(dims.end(), g2.begin(), g2.end());
      for (size_t v = 0; v < cx.vtab.size(); ++v) {
        size_t d = 0;
        for (auto s : s1[v]) cx.vtab[v].stride[d++] = s;
        for (auto s : s2[v]) cx.vtab[v].stride[d++] = s;
        for (; d < (size_t)kMaxDims; ++d) cx.vtab[v].stride[d] = 0;
      }
    }
    uint32_t vb = commit_views(cx);
    uint32_t src_first = commit_code(code, vb);
    const uint32_t fin_first = reduction_finish(e, rc);
    const uint32_t fin_len = last_finish_len;
    DTask t = blank(rc.kind);
    t.ndim = (uint8_t)dims.size();
    for (size_t d = 0; d < dims.size(); ++d) t.dims[d] = (uint32_t)dims[d];
    t.expr_first = src_first;
    t.expr_len = (uint32_t)code.size();
    t.fin_first = fin_first;
    t.fin_len = fin_len;
    t.split = rc.parts;
    t.kchunk = rc.kchunk;
    t.count = (float)rc.R;
    t.m = (uint32_t)rc.rows;
    t.k = (uint32_t)rc.R;
    if (r.opcode == "mean") t.flags |= F_MEAN;
    std::string desc = r.name + " (" + r.opcode + " " + std::to_string(rc.rows) + " outputs over " + std::to_string(rc.R) + ")";
    if (!e.side.empty()) {
      desc += " +side";
      for (int c : e.side) desc += " " + op(c).name;
      if (e.discard_root) desc += " (root discarded)";
    }
    if (rc.kind == T_RED_COLS) {
      t.width = (rc.rows % 8 == 0) ? 8 : 1;
      if (O.fast_epilogue && t.width == 8 && dims.size() == 2 && code.size() == 1 && code[0].op == VM_LOAD &&
          code[0].src == SRC_VIEW && code[0].rnd == RND_NONE && code[0].arg < cx.vtab.size()) {
        const DView& v = cx.vtab[code[0].arg];
        if (v.dtype != DT_I8 && v.stride[1] == 1) t.flags |= F_COLDIRECT;
      }
      // one part read directly: 8 column chunks x 32 row lanes per item
      if ((t.flags & F_COLDIRECT) && rc.parts == 1) t.flags |= F_COLLANES32;
      const uint32_t cols_per_item = (t.flags & F_COLLANES32) ? 64u : 32u * t.width;
      t.tiles_n = (uint32_t)((rc.rows + cols_per_item - 1) / cols_per_item);
      t.n_items = rc.rows == 0 ? 0 : t.tiles_n * rc.parts;
      if (t.flags & F_COLDIRECT) desc += " [rows summed directly]";
    } else {
      t.width = (dims.back() % 8 == 0 && rc.R % 8 == 0) ? 8 : 1;
      t.n_items = (uint32_t)(rc.rows * rc.parts);
    }
    if (rc.parts > 1) {
      t.flags |= F_PARTIAL;
      t.scratch = scratch_off.at((int)si);
      put(e.level, t, desc + " [" + std::to_string(rc.parts) + " partials]");
      DTask f = blank(T_RED_FINAL);
      f.m = (uint32_t)rc.rows;
      f.split = rc.parts;
      f.scratch = t.scratch;
      f.fin_first = fin_first;
      f.fin_len = fin_len;
      f.count = t.count;
      f.flags = t.flags & F_MEAN;
      f.tile = rc.kind == T_RED_COLS ? 1 : 0;  // partial layout: [parts][rows] (cols) or [rows][parts]
      f.n_items = (uint32_t)((rc.rows + kBlock - 1) / kBlock);
      if (rc.rows <= 32 && rc.parts >= 32) {
        // few outputs over many parts: a workgroup per output loads the parts
        // at once instead of one thread walking them
        f.flags |= F_ROWWG;
        f.n_items = (uint32_t)rc.rows;
      }
      put(e.level + 1, f, desc + " [combine]");
    } else {
      put(e.level, t, desc);
    }
  }

  // Safety net: no two tasks of a stage may touch overlapping regions unless
  // both only read (the pages' read/write hazard rule).
  void check_hazards() {
    struct R { int space; uint64_t lo, hi; };
    auto space_of = [&](int base) -> int {
      if (base >= n_in && base < n_in + n_out) {
        auto it = direct.find(base - n_in);
        if (it != direct.end()) return it->second;  // same memory as the input
      }
      return base;
    };
    std::map<int, std::vector<std::pair<std::vector<R>, std::vector<R>>>> per_level;
    std::map<int, std::vector<std::string>> per_level_name;
    std::map<std::string, const Entry*> writer;
    for (auto& e : sched)
      for (auto& w : e.writes_vals) writer[w] = &e;
    auto value_region = [&](const std::string& v) -> R {
      if (is_input(v)) return {input_idx[v], 0, ~0ull};
      const Loc& l = loc.at(v);
      if (l.base == ws_base) {
        uint64_t off = kHeaderBytes + arena_off.at(v);
        const Spec& pv = op(prod(v)).out;
        return {ws_base, off, off + std::max<uint64_t>(1, pv.numel() * dtype_size(pv.dtype))};
      }
      return {space_of(l.base), 0, ~0ull};
    };
    for (size_t i = 0; i < sched.size(); ++i) {
      const Entry& e = sched[i];
      std::vector<R> rd, wr;
      for (auto& v : e.reads_vals) rd.push_back(value_region(v));
      for (auto& t : e.reads_inputs) rd.push_back({input_idx[t], 0, ~0ull});
      for (auto& w : e.writes_vals) wr.push_back(value_region(w));
      if (e.kind != 0) wr.push_back({space_of(n_in + e.slot), 0, ~0ull});
      if (e.kind == 2)
        for (int wi : e.writes_inputs) wr.push_back({wi, 0, ~0ull});
      const std::string nm = e.kind == 0 ? op(e.op).name : ("out[" + std::to_string(e.slot) + "]");
      if (e.two_phase) {
        // phase 1 reads the operands and writes fp32 partials; phase 2 reads
        // the partials (and epilogue operands) and writes the values
        R s{ws_base, scratch_off.at((int)i), scratch_off.at((int)i) + scratch_bytes.at((int)i)};
        per_level[e.level].push_back({rd, {s}});
        per_level_name[e.level].push_back(nm);
        std::vector<R> rd2 = rd;
        rd2.push_back(s);
        per_level[e.level + 1].push_back({rd2, wr});
        per_level_name[e.level + 1].push_back(nm);
      } else {
        per_level[e.level].push_back({rd, wr});
        per_level_name[e.level].push_back(nm);
      }
    }
    auto ov = [](const R& a, const R& b) { return a.space == b.space && a.lo < b.hi && b.lo < a.hi; };
    for (auto& kv : per_level) {
      auto& v = kv.second;
      for (size_t a = 0; a < v.size(); ++a)
        for (size_t b = 0; b < v.size(); ++b) {
          if (a == b) continue;
          for (auto& w : v[a].second) {
            const std::string who = per_level_name[kv.first][a] + " vs " + per_level_name[kv.first][b];
            for (auto& w2 : v[b].second)
              if (ov(w, w2)) raise(TK_E_ARG, "internal: write/write hazard inside stage " + std::to_string(kv.first) + ": " + who);
            for (auto& r2 : v[b].first)
              if (ov(w, r2)) raise(TK_E_ARG, "internal: read/write hazard inside stage " + std::to_string(kv.first) + ": " + who);
          }
        }
    }
  }

  Plan run() {
    if (O.fuse_epilogues) {
      pass1();
      pass2();
    }
    choose_inline();
    build_input_use();
    build_schedule();
    prove_direct();
    pass3();
    bind_outputs();
    add_copies_and_commits();
    for (size_t i = 0; i < sched.size(); ++i) {
      sched[i].order = (int)i;
      sched[i].two_phase = two_phase_of(sched[i]);
    }
    collect_rw();
    level();
    fuse_column_sums();
    if (!colsum_host.empty()) level();
    size_scratch();
    plan_arena();
    check_hazards();
    for (size_t i = 0; i < sched.size(); ++i) {
      const Entry& e = sched[i];
      if (e.kind != 0) {
        emit_copy(e);
        continue;
      }
      const Op& o2 = op(e.op);
      if (o2.cls == OC_POINTWISE)
        emit_pointwise(e);
      else if (o2.cls == OC_REDUCE) {
        if (!colsum_host.count((int)i)) emit_reduction(i);
      } else {
        emit_contraction(i);
      }
    }
    return encode();
  }

  // One machine instruction as text (plan dumps).
  static std::string ins_text(const DIns& d) {
    static const char* names[] = {"?", "load", "add", "sub", "mul", "div", "neg", "relu", "square", "pow", "tb",
                                  "save", "store", "scale", "zero", "sqrt"};
    std::ostringstream o;
    o << (d.op < sizeof(names) / sizeof(names[0]) ? names[d.op] : "?");
    if (d.op == VM_STORE) o << "(v" << d.arg << ")";
    else if (d.op == VM_SAVE) o << "(s" << d.arg << ")";
    else if (d.src == SRC_VIEW) o << "(v" << d.arg << ")";
    else if (d.src == SRC_SLOT) o << "(s" << d.arg << ")";
    else if (d.src == SRC_SCALAR) o << "(" << d.s << ")";
    if (d.rev) o << "'";
    if (d.rnd == DT_BF16) o << ">bf16";
    else if (d.rnd == DT_F16) o << ">f16";
    return o.str();
  }

  Plan encode() {
    Plan pl;
    pl.n_in = n_in;
    pl.n_out = n_out;
    pl.ws_base = ws_base;
    pl.inputs = P.inputs;
    pl.outputs = P.outputs;
    pl.inplace = P.inplace;
    // drop empty levels
    std::vector<std::vector<DTask>> stages;
    std::vector<std::vector<std::string>> descs;
    for (size_t L = 0; L < stage_tasks.size(); ++L) {
      if (stage_tasks[L].empty()) continue;
      stages.push_back(stage_tasks[L]);
      descs.push_back(stage_desc[L]);
    }
    // Per stage: tasks, then the views and instructions they use, re-indexed
    // locally so the stage blob is self-contained.
    // A stage blob is staged whole in LDS by every workgroup; a level whose
    // descriptors exceed that buffer runs as several consecutive stages
    // (tasks of one level are independent, so any split is valid).
    struct Enc {
      DStage d;
      std::vector<uint8_t> blob;
      std::string dump;
      uint32_t items;
    };
    auto encode_group = [&](const std::vector<DTask>& group, const std::vector<std::string>& gdesc) -> Enc {
      std::vector<DTask> tk;
      std::vector<DView> sv;
      std::vector<DIns> si;
      std::map<uint32_t, uint16_t> vmap;
      auto mapv = [&](uint32_t g) -> uint16_t {
        auto it = vmap.find(g);
        if (it != vmap.end()) return it->second;
        uint16_t l = (uint16_t)sv.size();
        vmap[g] = l;
        sv.push_back(views.at(g));
        return l;
      };
      auto mapcode = [&](uint32_t first, uint32_t len) -> uint32_t {
        uint32_t at = (uint32_t)si.size();
        for (uint32_t i = 0; i < len; ++i) {
          DIns d = ins.at(first + i);
          if (d.src == SRC_VIEW || d.op == VM_STORE) d.arg = mapv(d.arg);
          si.push_back(d);
        }
        return at;
      };
      Enc e;
      e.items = 0;
      std::ostringstream gd;
      for (size_t t = 0; t < group.size(); ++t) {
        DTask task = group[t];
        set_divisors(task);
        task.item_begin = e.items;
        e.items += task.n_items;
        if (task.kind == T_GEMM_MFMA || task.kind == T_GEMM_SIMT || task.kind == T_GEMV_Q8) {
          task.va = mapv(task.va);
          task.vb = mapv(task.vb);
          if (task.kind == T_GEMV_Q8) task.vs = mapv(task.vs);
        }
        task.expr_first = task.expr_len ? mapcode(task.expr_first, task.expr_len) : 0;
        task.fin_first = task.fin_len ? mapcode(task.fin_first, task.fin_len) : 0;
        task.bs_first = task.bs_len ? mapcode(task.bs_first, task.bs_len) : 0;
        tk.push_back(task);
        gd << "  " << kind_name(task.kind) << " items=" << task.n_items << " : " << gdesc[t] << "\n";
        auto prog = [&](const char* what, uint32_t first, uint32_t len) {
          if (!len) return;
          gd << "    | " << what << ":";
          for (uint32_t i = 0; i < len; ++i) gd << " " << ins_text(si.at(first + i));
          gd << "\n";
        };
        prog("code", task.expr_first, task.expr_len);
        if (!(task.flags & F_FASTEPI)) prog("finish", task.fin_first, task.fin_len);
        prog("column sums", task.bs_first, task.bs_len);
      }
      DStage& d = e.d;
      d = DStage{};
      d.n_tasks = (uint32_t)tk.size();
      d.n_items = e.items;
      d.n_views = (uint32_t)sv.size();
      d.n_ins = (uint32_t)si.size();
      d.off_views = (uint32_t)align_up(tk.size() * sizeof(DTask), 16);
      d.off_ins = (uint32_t)align_up(d.off_views + sv.size() * sizeof(DView), 16);
      d.blob_bytes = (uint32_t)align_up(d.off_ins + si.size() * sizeof(DIns), 16);
      e.blob.assign(d.blob_bytes, 0);
      if (!tk.empty()) std::memcpy(e.blob.data(), tk.data(), tk.size() * sizeof(DTask));
      if (!sv.empty()) std::memcpy(e.blob.data() + d.off_views, sv.data(), sv.size() * sizeof(DView));
      if (!si.empty()) std::memcpy(e.blob.data() + d.off_ins, si.data(), si.size() * sizeof(DIns));
      e.dump = gd.str();
      return e;
    };
    std::vector<Enc> enc;
    for (size_t s = 0; s < stages.size(); ++s) {
      std::vector<DTask> group;
      std::vector<std::string> gdesc;
      for (size_t t = 0; t < stages[s].size(); ++t) {
        group.push_back(stages[s][t]);
        gdesc.push_back(descs[s][t]);
        if (encode_group(group, gdesc).d.blob_bytes <= kPlanLds) continue;
        if (group.size() == 1)
          raise(TK_E_UNSUPPORTED, "descriptors of one task exceed the " + std::to_string(kPlanLds) + "-byte stage buffer: " +
                                      descs[s][t]);
        group.pop_back();
        gdesc.pop_back();
        enc.push_back(encode_group(group, gdesc));
        group = {stages[s][t]};
        gdesc = {descs[s][t]};
      }
      if (!group.empty()) enc.push_back(encode_group(group, gdesc));
    }
    std::vector<DStage> ds;
    std::vector<std::vector<uint8_t>> blobs;
    int max_items = 0;
    size_t n_tasks_total = 0;
    std::ostringstream dump;
    for (size_t s = 0; s < enc.size(); ++s) {
      dump << "stage " << s << ":\n" << enc[s].dump;
      ds.push_back(enc[s].d);
      blobs.push_back(enc[s].blob);
      max_items = std::max<int>(max_items, (int)enc[s].items);
      n_tasks_total += enc[s].d.n_tasks;
    }
    dump << "workspace: " << kHeaderBytes << " header + " << arena_bytes << " arena bytes\n";
    for (auto& kv : arena_off) dump << "  arena " << kv.first << " @" << kv.second << "\n";
    for (auto& kv : bound) dump << "  bound " << kv.first << " -> out[" << kv.second << "]\n";
    for (auto& kv : direct) dump << "  direct in-place out[" << kv.first << "] -> in[" << kv.second << "]\n";
    // serialize: header | stage table | blobs
    DHeader h{};
    h.magic = kPlanMagic;
    h.n_stages = (uint32_t)ds.size();
    h.off_stages = (uint32_t)align_up(sizeof(DHeader), 64);
    uint32_t off = (uint32_t)align_up(h.off_stages + ds.size() * sizeof(DStage), 64);
    for (size_t s = 0; s < ds.size(); ++s) {
      ds[s].blob_off = off;
      off = (uint32_t)align_up(off + ds[s].blob_bytes, 64);
      h.max_blob = std::max(h.max_blob, ds[s].blob_bytes);
    }
    h.bytes = off;
    pl.bytes.assign(off, 0);
    std::memcpy(pl.bytes.data(), &h, sizeof(h));
    if (!ds.empty()) std::memcpy(pl.bytes.data() + h.off_stages, ds.data(), ds.size() * sizeof(DStage));
    for (size_t s = 0; s < ds.size(); ++s)
      if (!blobs[s].empty()) std::memcpy(pl.bytes.data() + ds[s].blob_off, blobs[s].data(), blobs[s].size());
    pl.n_stages = (int)ds.size();
    pl.max_items = max_items;
    pl.workspace_bytes = kHeaderBytes + align_up(arena_bytes, kAlign);
    // arena views address the workspace with 32-bit element indices
    if (pl.workspace_bytes > (uint64_t)0x7fffffff)
      raise(TK_E_UNSUPPORTED, "workspace above 2 GiB (" + std::to_string(pl.workspace_bytes) + " bytes)");
    pl.dump = dump.str();
    // statistics
    tk_stats& s = pl.stats;
    s = st;
    s.workspace_bytes = pl.workspace_bytes;
    s.n_stages = (int32_t)ds.size();
    s.grid_barriers = std::max(0, (int32_t)ds.size() - 1);
    s.n_tasks = (int32_t)n_tasks_total;
    s.inlined_ops = (int32_t)inlined.size();
    int mat = 0, fe = 0, se = 0, fu = 0;
    for (auto& e : sched) {
      if (e.kind != 0) continue;
      mat++;
      if (!e.chain.empty() && !e.update) fe++;
      if (e.update) fu++;
      // side programs: those writing other values than in-place updates count
      // as side epilogues, each directly committed update as a fused update
      bool other = false;
      for (int c : e.side) {
        const std::string& b = op(c).out.buf;
        if (!aliased.count(b) && side_stored(e, c)) other = true;
        if (aliased.count(b))
          for (auto& kv : direct)
            if (P.outputs[kv.first].buf == b) fu++;
      }
      if (other) se++;
    }
    s.materialized_ops = mat;
    s.fused_epilogues = fe;
    s.side_epilogues = se;
    s.fused_updates = fu;
    s.direct_outputs = (int32_t)bound.size();
    s.direct_state_commits = (int32_t)direct.size();
    s.staged_commits = (int32_t)(P.inplace.size() - direct.size());
    s.max_work_items = max_items;
    s.num_cus = O.num_cus;
    return pl;
  }
};

}  // namespace

Plan schedule_program(const Program& p, const Options& o) {
  Builder b(p, o);
  return b.run();
}

}  // namespace tk
