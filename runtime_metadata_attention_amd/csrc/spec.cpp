// spec.cpp -- MaskSpec parsing and symbolic lowering to visible intervals.
//
// CompileMask paper summary, section 3.2.1 "Mask Specification": a MaskSpec
// groups query rows into Regions; each Region has a row guard and a
// visibility rule, kept apart so that the spec can be reused while batch
// boundaries change.  Section 3.2.2 "Symbolic Lowering to Visible Intervals":
// each rule goes through AST construction, DNF normalisation, interval
// extraction and canonicalisation, and the compiler keeps as many interval
// slots as the rule needs over the whole Region (two for [0,b) u [s(i),i+1),
// which cannot be merged across the Region).  Forward and backward use
// separate rules so that each table follows its pass's traversal (section
// 3.3 "Online Efficient Mask Attention Execution").
//
// Text form (newlines are insignificant; `#` starts a comment):
//   mask NAME                 optional name
//   param P, h, ...           per-sample scalars, in metadata order
//   refs R                    references per segment carried by the metadata
//   forward                   rules over query rows i; free variable j (keys)
//   backward                  rules over key columns j; free variable i (rows)
//   region NAME : GUARD => RULE
// GUARD and RULE are boolean formulas: `&`, `|`, `!`, parentheses, `true`,
// `false`, comparisons (< <= > >= == !=) of integer expressions, `x in [a, b)`
// (or `[a, b]`), `x in S`, and `exists k ( ... )` over the segments of the
// sample.  Integer expressions: literals, i, j, N, params, start(S), end(S),
// +, -.  Segment expressions S: seg(i) / seg(j) (the segment holding that
// index), ref(S, r) (S's r-th reference), or the exists variable.  A segment
// expression used as a number is its id (so `ref(k,0) == seg(j)` compares ids).
#include <algorithm>
#include <atomic>
#include <cctype>
#include <map>
#include <memory>
#include <sstream>
#include <stdexcept>
#include <tuple>

#include "internal.h"

namespace cm {
namespace {

// ---------------------------------------------------------------- terms

enum Root { R_IDX = 0, R_K = 1, R_FREE = 2 };
enum Kind { K_IDX, K_FREE, K_N, K_SCALAR, K_START, K_END, K_SEGID };

struct Sel {
  int root = R_IDX;
  std::vector<int> hops;
  bool operator<(const Sel& o) const { return std::tie(root, hops) < std::tie(o.root, o.hops); }
  bool operator==(const Sel& o) const { return root == o.root && hops == o.hops; }
};

struct Base {
  int kind = K_IDX;
  int arg = 0;  // scalar index
  Sel sel;      // segment selector for START / END / SEGID
  bool operator<(const Base& o) const { return std::tie(kind, arg, sel) < std::tie(o.kind, o.arg, o.sel); }
  bool operator==(const Base& o) const { return kind == o.kind && arg == o.arg && sel == o.sel; }
};

struct Lin {
  std::map<Base, int64_t> c;
  int64_t k = 0;
  Lin& add(const Lin& o, int64_t m) {
    for (auto& kv : o.c) {
      int64_t& v = c[kv.first];
      v += m * kv.second;
      if (v == 0) c.erase(kv.first);
    }
    k += m * o.k;
    return *this;
  }
  static Lin constant(int64_t v) { Lin l; l.k = v; return l; }
  static Lin base(const Base& b) { Lin l; l.c[b] = 1; return l; }
  bool operator<(const Lin& o) const { return std::tie(c, k) < std::tie(o.c, o.k); }
  bool operator==(const Lin& o) const { return c == o.c && k == o.k; }
  int64_t coef(int kind) const {
    int64_t s = 0;
    for (auto& kv : c) if (kv.first.kind == kind) s += kv.second;
    return s;
  }
  bool uses_root(int root) const {
    for (auto& kv : c)
      if ((kv.first.kind == K_START || kv.first.kind == K_END || kv.first.kind == K_SEGID) && kv.first.sel.root == root)
        return true;
    return false;
  }
};

enum Op { LT, LE, GT, GE, EQ, NE };
Op negate(Op o) {
  switch (o) { case LT: return GE; case LE: return GT; case GT: return LE; case GE: return LT; case EQ: return NE; default: return EQ; }
}
Op flip(Op o) {  // a op b  <=>  b flip(op) a
  switch (o) { case LT: return GT; case LE: return GE; case GT: return LT; case GE: return LE; default: return o; }
}

// ---------------------------------------------------------------- AST

struct BNode {
  enum T { AND, OR, NOT, EXISTS, CMP, TRUE_, FALSE_ } t;
  std::vector<std::unique_ptr<BNode>> kids;
  Op op = LT;
  Lin lin;  // CMP: lin op 0
  explicit BNode(T t_) : t(t_) {}
};
using BP = std::unique_ptr<BNode>;

BP mk(BNode::T t) { return BP(new BNode(t)); }
BP mk2(BNode::T t, BP a, BP b) {
  BP n = mk(t);
  n->kids.push_back(std::move(a));
  n->kids.push_back(std::move(b));
  return n;
}
BP cmp(Op op, const Lin& l, const Lin& r) {
  BP n = mk(BNode::CMP);
  n->op = op;
  n->lin = l;
  n->lin.add(r, -1);
  return n;
}

struct SpecError : std::runtime_error {
  using std::runtime_error::runtime_error;
};

// ---------------------------------------------------------------- lexer

struct Tok {
  enum Kind { ID, NUM, OP, END } kind;
  std::string s;
  int64_t v = 0;
  int line = 0;
};

std::vector<Tok> lex(const std::string& text) {
  std::vector<Tok> out;
  int line = 1;
  size_t p = 0;
  while (p < text.size()) {
    char ch = text[p];
    if (ch == '\n') { ++line; ++p; continue; }
    if (std::isspace((unsigned char)ch)) { ++p; continue; }
    if (ch == '#') { while (p < text.size() && text[p] != '\n') ++p; continue; }
    if (std::isalpha((unsigned char)ch) || ch == '_') {
      size_t q = p;
      while (q < text.size() && (std::isalnum((unsigned char)text[q]) || text[q] == '_')) ++q;
      out.push_back({Tok::ID, text.substr(p, q - p), 0, line});
      p = q;
      continue;
    }
    if (std::isdigit((unsigned char)ch)) {
      size_t q = p;
      int64_t v = 0;
      while (q < text.size() && std::isdigit((unsigned char)text[q])) {
        v = v * 10 + (text[q] - '0');
        if (v > (int64_t(1) << 40)) throw SpecError("line " + std::to_string(line) + ": integer too large");
        ++q;
      }
      out.push_back({Tok::NUM, text.substr(p, q - p), v, line});
      p = q;
      continue;
    }
    static const char* two[] = {"<=", ">=", "==", "!=", "=>", "&&", "||"};
    bool done = false;
    for (const char* t : two) {
      if (text.compare(p, 2, t) == 0) {
        std::string s(t);
        if (s == "&&") s = "&";
        if (s == "||") s = "|";
        out.push_back({Tok::OP, s, 0, line});
        p += 2;
        done = true;
        break;
      }
    }
    if (done) continue;
    if (std::string("<>()[],:+-&|!").find(ch) != std::string::npos) {
      out.push_back({Tok::OP, std::string(1, ch), 0, line});
      ++p;
      continue;
    }
    throw SpecError("line " + std::to_string(line) + ": unexpected character '" + std::string(1, ch) + "'");
  }
  out.push_back({Tok::END, "", 0, line});
  return out;
}

// ---------------------------------------------------------------- parser

bool is_stmt_keyword(const std::string& s) {
  return s == "mask" || s == "param" || s == "refs" || s == "forward" || s == "backward" || s == "region";
}

struct RegionAst {
  std::string name;
  BP guard, rule;
  int line;
};

struct Parser {
  std::vector<Tok> t;
  size_t p = 0;
  std::vector<std::string> params;
  int n_refs = 0;
  std::string idx_var, free_var, exists_var;

  const Tok& cur() const { return t[p]; }
  bool is_op(const char* s) const { return t[p].kind == Tok::OP && t[p].s == s; }
  bool is_id(const char* s) const { return t[p].kind == Tok::ID && t[p].s == s; }
  [[noreturn]] void err(const std::string& m) const {
    throw SpecError("line " + std::to_string(t[p].line) + ": " + m +
                    (t[p].kind == Tok::END ? " (at end of text)" : " (at '" + t[p].s + "')"));
  }
  void expect_op(const char* s) {
    if (!is_op(s)) err(std::string("expected '") + s + "'");
    ++p;
  }
  std::string expect_id() {
    if (t[p].kind != Tok::ID) err("expected a name");
    return t[p++].s;
  }
  int64_t expect_num() {
    if (t[p].kind != Tok::NUM) err("expected an integer");
    return t[p++].v;
  }

  // segment expression -> selector
  Sel parse_seg() {
    if (is_id("seg")) {
      ++p;
      expect_op("(");
      Lin x = parse_arith();
      expect_op(")");
      Sel s;
      if (x.k == 0 && x.c.size() == 1 && x.c.begin()->second == 1 && x.c.begin()->first.kind == K_IDX) s.root = R_IDX;
      else if (x.k == 0 && x.c.size() == 1 && x.c.begin()->second == 1 && x.c.begin()->first.kind == K_FREE) s.root = R_FREE;
      else err("seg() takes the row or column index itself");
      return s;
    }
    if (is_id("ref")) {
      ++p;
      expect_op("(");
      Sel s = parse_seg();
      expect_op(",");
      int64_t r = expect_num();
      expect_op(")");
      if (r >= n_refs) err("reference index " + std::to_string(r) + " >= refs " + std::to_string(n_refs));
      if (s.hops.size() >= 2) err("at most two nested ref()");
      s.hops.push_back((int)r);
      return s;
    }
    if (!exists_var.empty() && t[p].kind == Tok::ID && t[p].s == exists_var) {
      ++p;
      Sel s;
      s.root = R_K;
      return s;
    }
    err("expected a segment expression: seg(x), ref(S, r) or the exists variable");
  }

  bool at_seg_start() const {
    return is_id("seg") || is_id("ref") || (!exists_var.empty() && t[p].kind == Tok::ID && t[p].s == exists_var);
  }

  Lin parse_factor() {
    if (t[p].kind == Tok::NUM) return Lin::constant(t[p++].v);
    if (is_op("(")) {
      ++p;
      Lin l = parse_arith();
      expect_op(")");
      return l;
    }
    if (is_id("start") || is_id("end")) {
      bool st = is_id("start");
      ++p;
      expect_op("(");
      Sel s = parse_seg();
      expect_op(")");
      if (s.root == R_FREE) err("start()/end() of seg() of the free variable is not an endpoint");
      Base b;
      b.kind = st ? K_START : K_END;
      b.sel = s;
      return Lin::base(b);
    }
    if (at_seg_start()) {
      Base b;
      b.kind = K_SEGID;
      b.sel = parse_seg();
      return Lin::base(b);
    }
    if (t[p].kind == Tok::ID) {
      if (is_stmt_keyword(t[p].s)) err("unexpected keyword; the expression is incomplete");
      std::string id = t[p++].s;
      Base b;
      if (id == idx_var) b.kind = K_IDX;
      else if (id == free_var) b.kind = K_FREE;
      else if (id == "N") b.kind = K_N;
      else {
        auto it = std::find(params.begin(), params.end(), id);
        if (it == params.end()) { --p; err("unknown name '" + id + "'"); }
        b.kind = K_SCALAR;
        b.arg = int(it - params.begin());
      }
      return Lin::base(b);
    }
    err("expected an integer expression");
  }

  Lin parse_term() {
    if (is_op("-")) { ++p; Lin l; l.add(parse_term(), -1); return l; }
    if (is_op("+")) { ++p; return parse_term(); }
    return parse_factor();
  }

  Lin parse_arith() {
    Lin l = parse_term();
    while (is_op("+") || is_op("-")) {
      int m = is_op("+") ? 1 : -1;
      ++p;
      l.add(parse_term(), m);
    }
    return l;
  }

  BP parse_atom() {
    Lin x = parse_arith();
    if (is_id("in")) {
      ++p;
      if (is_op("[")) {
        ++p;
        Lin a = parse_arith();
        expect_op(",");
        Lin b = parse_arith();
        bool closed;
        if (is_op(")")) closed = false;
        else if (is_op("]")) closed = true;
        else err("expected ')' or ']'");
        ++p;
        return mk2(BNode::AND, cmp(GE, x, a), cmp(closed ? LE : LT, x, b));
      }
      Sel s = parse_seg();
      if (s.root == R_FREE) err("'in' needs a segment that does not depend on the free variable");
      Base st, en;
      st.kind = K_START; st.sel = s;
      en.kind = K_END; en.sel = s;
      return mk2(BNode::AND, cmp(GE, x, Lin::base(st)), cmp(LT, x, Lin::base(en)));
    }
    static const std::pair<const char*, Op> ops[] = {{"<", LT}, {"<=", LE}, {">", GT}, {">=", GE}, {"==", EQ}, {"!=", NE}};
    for (auto& o : ops) {
      if (is_op(o.first)) {
        ++p;
        Lin y = parse_arith();
        return cmp(o.second, x, y);
      }
    }
    err("expected a comparison or 'in'");
  }

  BP parse_primary() {
    if (is_id("true")) { ++p; return mk(BNode::TRUE_); }
    if (is_id("false")) { ++p; return mk(BNode::FALSE_); }
    if (is_op("(")) {
      // a parenthesised formula, unless it is the start of an integer expression
      size_t save = p;
      std::string save_var = exists_var;
      try {
        ++p;
        BP b = parse_or();
        expect_op(")");
        if (!(is_op("<") || is_op("<=") || is_op(">") || is_op(">=") || is_op("==") || is_op("!=") ||
              is_op("+") || is_op("-") || is_id("in")))
          return b;
      } catch (const SpecError&) {
      }
      p = save;
      exists_var = save_var;
    }
    return parse_atom();
  }

  BP parse_unary() {
    if (is_op("!")) {
      ++p;
      BP n = mk(BNode::NOT);
      n->kids.push_back(parse_unary());
      return n;
    }
    if (is_id("exists")) {
      ++p;
      if (!exists_var.empty()) err("nested exists");
      std::string v = expect_id();
      if (v == idx_var || v == free_var || v == "N" || std::find(params.begin(), params.end(), v) != params.end())
        err("exists variable shadows another name");
      expect_op("(");
      exists_var = v;
      BP body = parse_or();
      exists_var.clear();
      expect_op(")");
      BP n = mk(BNode::EXISTS);
      n->kids.push_back(std::move(body));
      return n;
    }
    return parse_primary();
  }

  BP parse_and() {
    BP l = parse_unary();
    while (is_op("&")) { ++p; l = mk2(BNode::AND, std::move(l), parse_unary()); }
    return l;
  }

  BP parse_or() {
    BP l = parse_and();
    while (is_op("|")) { ++p; l = mk2(BNode::OR, std::move(l), parse_and()); }
    return l;
  }
};

// ---------------------------------------------------------------- lowering

struct Cond {
  Op op;  // LT, LE, EQ, NE only after normalisation
  Lin lin;
  bool operator<(const Cond& o) const { return std::tie(op, lin) < std::tie(o.op, o.lin); }
  bool operator==(const Cond& o) const { return op == o.op && lin == o.lin; }
};

struct Conj {
  bool family = false;
  std::vector<Lin> lo, hi;
  std::vector<std::vector<Cond>> conds;  // OR of ANDs; empty = unconditional
};

// negation normal form: push NOT down to the atoms
BP nnf(BP n, bool neg) {
  switch (n->t) {
    case BNode::NOT: return nnf(std::move(n->kids[0]), !neg);
    case BNode::TRUE_: return neg ? mk(BNode::FALSE_) : std::move(n);
    case BNode::FALSE_: return neg ? mk(BNode::TRUE_) : std::move(n);
    case BNode::CMP: if (neg) n->op = negate(n->op); return n;
    case BNode::EXISTS:
      if (neg) throw SpecError("a negated exists cannot be lowered to intervals");
      n->kids[0] = nnf(std::move(n->kids[0]), false);
      return n;
    case BNode::AND:
    case BNode::OR: {
      BNode::T t = n->t;
      if (neg) t = (t == BNode::AND) ? BNode::OR : BNode::AND;
      BP m = mk(t);
      for (auto& k : n->kids) m->kids.push_back(nnf(std::move(k), neg));
      return m;
    }
  }
  return n;
}

void check_term(const Lin& l, const char* what) {
  if (l.c.size() > 2) throw SpecError(std::string(what) + " has more than two symbolic parts");
  for (auto& kv : l.c) {
    if (kv.second != 1 && kv.second != -1) throw SpecError(std::string(what) + " multiplies a symbol");
    if (kv.first.kind == K_FREE) throw SpecError(std::string(what) + " depends on the free variable");
    if (kv.first.sel.root == R_FREE && (kv.first.kind == K_START || kv.first.kind == K_END || kv.first.kind == K_SEGID))
      throw SpecError(std::string(what) + " uses seg() of the free variable");
  }
  if (l.k > INT32_MAX || l.k < INT32_MIN) throw SpecError(std::string(what) + " constant out of range");
}

Cond make_cond(Op op, Lin lin) {
  if (op == GT) { Lin m; m.add(lin, -1); return make_cond(LT, m); }
  if (op == GE) { Lin m; m.add(lin, -1); return make_cond(LE, m); }
  check_term(lin, "a condition");
  return Cond{op, lin};
}

using DNF = std::vector<Conj>;

Conj conj_and(const Conj& a, const Conj& b) {
  if (a.family && b.family) throw SpecError("two exists in one conjunction");
  Conj c;
  c.family = a.family || b.family;
  c.lo = a.lo; c.lo.insert(c.lo.end(), b.lo.begin(), b.lo.end());
  c.hi = a.hi; c.hi.insert(c.hi.end(), b.hi.begin(), b.hi.end());
  // conds: (OR of A) AND (OR of B) = OR over pairs
  if (a.conds.empty()) c.conds = b.conds;
  else if (b.conds.empty()) c.conds = a.conds;
  else
    for (auto& x : a.conds)
      for (auto& y : b.conds) {
        std::vector<Cond> z = x;
        z.insert(z.end(), y.begin(), y.end());
        c.conds.push_back(z);
      }
  return c;
}

DNF leaf_bound(bool is_lo, const Lin& x) {
  check_term(x, "an endpoint");
  Conj c;
  (is_lo ? c.lo : c.hi).push_back(x);
  return {c};
}

DNF dnf_or(DNF a, const DNF& b) {
  a.insert(a.end(), b.begin(), b.end());
  return a;
}

DNF dnf_and(const DNF& a, const DNF& b) {
  DNF out;
  for (auto& x : a)
    for (auto& y : b) out.push_back(conj_and(x, y));
  if (out.size() > 64) throw SpecError("rule expands to more than 64 conjunctions");
  return out;
}

// one comparison atom -> DNF of bounds on the free variable and conditions
DNF lower_cmp(Op op, const Lin& lin, bool allow_free) {
  // seg(free) == S  /  seg(free) != S
  for (auto& kv : lin.c) {
    const Base& b = kv.first;
    if (b.kind == K_SEGID && b.sel.root == R_FREE) {
      if (!allow_free) throw SpecError("a guard may not use the free variable");
      if (!b.sel.hops.empty()) throw SpecError("ref() of seg() of the free variable is not supported");
      if (op != EQ && op != NE) throw SpecError("seg() of the free variable can only be compared with == or !=");
      Lin rest = lin;
      int64_t m = kv.second;
      rest.c.erase(b);
      if (rest.k != 0 || rest.c.size() != 1 || rest.c.begin()->first.kind != K_SEGID || rest.c.begin()->second != -m)
        throw SpecError("seg() of the free variable must be compared with one segment");
      Sel s = rest.c.begin()->first.sel;
      if (s.root == R_FREE) throw SpecError("seg(free) compared with itself");
      Base st, en;
      st.kind = K_START; st.sel = s;
      en.kind = K_END; en.sel = s;
      if (op == EQ) return dnf_and(leaf_bound(true, Lin::base(st)), leaf_bound(false, Lin::base(en)));
      return dnf_or(leaf_bound(false, Lin::base(st)), leaf_bound(true, Lin::base(en)));
    }
  }
  int64_t c = lin.coef(K_FREE);
  if (c == 0) {
    Conj cj;
    cj.conds.push_back({make_cond(op, lin)});
    return {cj};
  }
  if (!allow_free) throw SpecError("a guard may not use the free variable");
  if (c != 1 && c != -1) throw SpecError("the free variable must appear with coefficient +1 or -1");
  Lin rest = lin;
  for (auto it = rest.c.begin(); it != rest.c.end();)
    it = (it->first.kind == K_FREE) ? rest.c.erase(it) : std::next(it);
  // c*F + rest op 0  ->  F op' X
  Lin X;
  Op o = op;
  if (c == 1) X.add(rest, -1);
  else { X = rest; o = flip(op); }
  Lin X1 = X;
  X1.k += 1;
  switch (o) {
    case LT: return leaf_bound(false, X);
    case LE: return leaf_bound(false, X1);
    case GT: return leaf_bound(true, X1);
    case GE: return leaf_bound(true, X);
    case EQ: return dnf_and(leaf_bound(true, X), leaf_bound(false, X1));
    case NE: return dnf_or(leaf_bound(false, X), leaf_bound(true, X1));
  }
  return {};
}

DNF to_dnf(const BNode* n, bool allow_free) {
  switch (n->t) {
    case BNode::TRUE_: return {Conj{}};
    case BNode::FALSE_: return {};
    case BNode::CMP: return lower_cmp(n->op, n->lin, allow_free);
    case BNode::AND: {
      DNF d = to_dnf(n->kids[0].get(), allow_free);
      for (size_t i = 1; i < n->kids.size(); ++i) d = dnf_and(d, to_dnf(n->kids[i].get(), allow_free));
      return d;
    }
    case BNode::OR: {
      DNF d;
      for (auto& k : n->kids) d = dnf_or(d, to_dnf(k.get(), allow_free));
      return d;
    }
    case BNode::EXISTS: {
      DNF d = to_dnf(n->kids[0].get(), allow_free);
      for (auto& c : d) {
        if (c.family) throw SpecError("nested exists");
        c.family = true;
      }
      return d;
    }
    case BNode::NOT: throw SpecError("internal: NOT after NNF");
  }
  return {};
}

// ---------------------------------------------------------------- prover
//
// Difference constraints x - y <= w over the symbolic bases of one Region,
// closed with Floyd-Warshall; t1 <= t2 is proved when dist(node(t2) ->
// node(t1)) <= const(t2) - const(t1).  Facts: 0 <= idx <= N - 1; segment
// boundaries lie in [0, N] with start(S) <= end(S); the segment holding the
// index contains it; and the Region's guard atoms.

struct Prover {
  std::vector<Base> nodes;  // node 0 = the constant zero
  std::vector<std::vector<int64_t>> d;
  static constexpr int64_t INF = int64_t(1) << 60;

  int node(const Base& b) {
    for (size_t i = 1; i < nodes.size(); ++i) if (nodes[i] == b) return int(i);
    nodes.push_back(b);
    return int(nodes.size() - 1);
  }
  static bool single(const Lin& l) { return l.c.size() == 0 || (l.c.size() == 1 && l.c.begin()->second == 1); }
  static bool orderable(const Base& b) { return b.kind != K_SEGID && b.kind != K_FREE; }

  void collect(const Lin& l) {
    for (auto& kv : l.c) if (orderable(kv.first)) node(kv.first);
  }

  void build(const std::vector<Cond>& guard, const std::vector<Conj>& slots) {
    nodes.assign(1, Base{});
    Base idx; idx.kind = K_IDX;
    Base nn; nn.kind = K_N;
    node(idx); node(nn);
    for (auto& g : guard) collect(g.lin);
    for (auto& s : slots) { for (auto& l : s.lo) collect(l); for (auto& l : s.hi) collect(l); }
    // add the partner boundary of every segment boundary
    size_t n0 = nodes.size();
    for (size_t i = 1; i < n0; ++i) {
      if (nodes[i].kind == K_START || nodes[i].kind == K_END) {
        Base o = nodes[i];
        o.kind = (o.kind == K_START) ? K_END : K_START;
        node(o);
      }
    }
    size_t n = nodes.size();
    d.assign(n, std::vector<int64_t>(n, INF));
    for (size_t i = 0; i < n; ++i) d[i][i] = 0;
    auto le = [&](int x, int y, int64_t w) {  // x - y <= w : edge y -> x
      d[y][x] = std::min(d[y][x], w);
    };
    int I = node(idx), NN = node(nn);
    le(0, I, 0);        // 0 <= idx
    le(I, NN, -1);      // idx <= N - 1
    for (size_t i = 1; i < n; ++i) {
      const Base& b = nodes[i];
      if (b.kind == K_START || b.kind == K_END) {
        le(0, int(i), 0);        // 0 <= boundary
        le(int(i), NN, 0);       // boundary <= N
      }
      if (b.kind == K_START) {
        Base e = b; e.kind = K_END;
        le(int(i), node(e), 0);  // start <= end
        if (b.sel.root == R_IDX && b.sel.hops.empty()) {
          le(int(i), I, 0);      // start(seg(idx)) <= idx
          le(I, node(e), -1);    // idx + 1 <= end(seg(idx))
        }
      }
    }
    for (auto& g : guard) {
      // g.lin op 0 with at most two orderable bases of coefficient +-1
      const Lin& l = g.lin;
      int pos = 0, neg = 0, np = 0, nn2 = 0;
      bool ok = true;
      for (auto& kv : l.c) {
        if (!orderable(kv.first)) { ok = false; break; }
        if (kv.second == 1) { pos = node(kv.first); ++np; }
        else if (kv.second == -1) { neg = node(kv.first); ++nn2; }
        else ok = false;
      }
      if (!ok || np > 1 || nn2 > 1) continue;
      // pos - neg + k op 0   (missing side = zero node)
      int64_t k = l.k;
      if (g.op == LT) le(pos, neg, -k - 1);
      else if (g.op == LE) le(pos, neg, -k);
      else if (g.op == EQ) { le(pos, neg, -k); le(neg, pos, k); }
    }
    n = nodes.size();
    for (auto& row : d) row.resize(n, INF);
    while (d.size() < n) { d.emplace_back(n, INF); d.back()[d.size() - 1] = 0; }
    for (size_t k = 0; k < n; ++k)
      for (size_t i = 0; i < n; ++i)
        if (d[i][k] < INF)
          for (size_t j = 0; j < n; ++j)
            if (d[k][j] < INF && d[i][k] + d[k][j] < d[i][j]) d[i][j] = d[i][k] + d[k][j];
  }

  int find(const Lin& l) const {
    if (l.c.empty()) return 0;
    const Base& b = l.c.begin()->first;
    for (size_t i = 1; i < nodes.size(); ++i) if (nodes[i] == b) return int(i);
    return -1;
  }
  // prove a <= b
  bool le(const Lin& a, const Lin& b) const {
    if (!single(a) || !single(b)) return false;
    int x = find(a), y = find(b);
    if (x < 0 || y < 0) return false;
    if (a.c.size() == 1 && !orderable(a.c.begin()->first)) return false;
    if (b.c.size() == 1 && !orderable(b.c.begin()->first)) return false;
    return d[y][x] < INF && d[y][x] <= b.k - a.k;
  }
};

// evaluate a condition with no symbols
int const_cond(const Cond& c) {  // -1 unknown, 0 false, 1 true
  if (!c.lin.c.empty()) return -1;
  int64_t v = c.lin.k;
  switch (c.op) {
    case LT: return v < 0; case LE: return v <= 0; case EQ: return v == 0; case NE: return v != 0;
    default: return -1;
  }
}

Lin lin_zero() { return Lin::constant(0); }
Lin lin_n() { Base b; b.kind = K_N; return Lin::base(b); }

// Endpoints are clamped to [0, N] when evaluated, so clamp(a) <= clamp(b)
// also holds when a <= 0 or b >= N.
bool le_clamped(const Prover& pv, const Lin& a, const Lin& b) {
  return pv.le(a, b) || pv.le(a, lin_zero()) || pv.le(lin_n(), b);
}

bool canonicalise_once(std::vector<Conj>& slots, const Prover& pv) {
  bool changed = false;
  std::vector<Conj> out;
  for (auto& s0 : slots) {
    Conj s = s0;
    // constant conditions
    if (!s.conds.empty()) {
      std::vector<std::vector<Cond>> keep;
      bool always = false;
      for (auto& cj : s.conds) {
        std::vector<Cond> k;
        bool dead = false;
        for (auto& c : cj) {
          int v = const_cond(c);
          if (v == 0) { dead = true; break; }
          if (v == -1) k.push_back(c);
        }
        if (dead) continue;
        std::sort(k.begin(), k.end());
        k.erase(std::unique(k.begin(), k.end()), k.end());
        if (k.empty()) always = true;
        keep.push_back(k);
      }
      std::sort(keep.begin(), keep.end());
      keep.erase(std::unique(keep.begin(), keep.end()), keep.end());
      if (keep.empty()) { changed = true; continue; }  // never true
      if (always) keep.clear();
      if (keep != s.conds) changed = true;
      s.conds = keep;
    }
    // redundant bounds
    auto prune = [&](std::vector<Lin>& v, bool is_lo) {
      std::sort(v.begin(), v.end());
      v.erase(std::unique(v.begin(), v.end()), v.end());
      for (size_t a = 0; a < v.size();) {
        bool red = is_lo ? pv.le(v[a], lin_zero()) : pv.le(lin_n(), v[a]);
        for (size_t b = 0; b < v.size() && !red; ++b)
          if (b != a) red = is_lo ? pv.le(v[a], v[b]) : pv.le(v[b], v[a]);
        if (red) { v.erase(v.begin() + a); changed = true; } else ++a;
      }
    };
    prune(s.lo, true);
    prune(s.hi, false);
    // provably empty
    bool empty = false;
    std::vector<Lin> los = s.lo.empty() ? std::vector<Lin>{lin_zero()} : s.lo;
    std::vector<Lin> his = s.hi.empty() ? std::vector<Lin>{lin_n()} : s.hi;
    for (auto& h : his) for (auto& l : los) if (le_clamped(pv, h, l)) empty = true;
    if (empty) { changed = true; continue; }
    out.push_back(s);
  }
  // same interval under different conditions -> one slot
  for (size_t a = 0; a < out.size(); ++a) {
    for (size_t b = a + 1; b < out.size();) {
      if (out[a].family == out[b].family && out[a].lo == out[b].lo && out[a].hi == out[b].hi) {
        if (out[a].conds.empty() || out[b].conds.empty()) out[a].conds.clear();
        else out[a].conds.insert(out[a].conds.end(), out[b].conds.begin(), out[b].conds.end());
        out.erase(out.begin() + b);
        changed = true;
      } else ++b;
    }
  }
  // plain unconditional intervals: containment and provable adjacency
  auto plain = [](const Conj& c) { return !c.family && c.conds.empty() && c.lo.size() <= 1 && c.hi.size() <= 1; };
  for (size_t a = 0; a < out.size(); ++a) {
    for (size_t b = 0; b < out.size();) {
      if (a == b || !plain(out[a]) || !plain(out[b])) { ++b; continue; }
      Lin A = out[a].lo.empty() ? lin_zero() : out[a].lo[0], Bh = out[a].hi.empty() ? lin_n() : out[a].hi[0];
      Lin C = out[b].lo.empty() ? lin_zero() : out[b].lo[0], D = out[b].hi.empty() ? lin_n() : out[b].hi[0];
      bool contained = le_clamped(pv, A, C) && le_clamped(pv, D, Bh);
      bool adjacent = le_clamped(pv, A, C) && le_clamped(pv, C, Bh) && le_clamped(pv, Bh, D);
      if (contained || adjacent) {
        if (adjacent && !contained) {
          out[a].hi.clear();
          if (!(pv.le(lin_n(), D))) out[a].hi.push_back(D);
        }
        out.erase(out.begin() + b);
        if (b < a) --a;
        changed = true;
        b = 0;
      } else ++b;
    }
  }
  slots = out;
  return changed;
}

struct RegionIR {
  std::string name;
  std::vector<Cond> guard;
  std::vector<Conj> slots;
};

// ---------------------------------------------------------------- encoding

int enc_sel(const Sel& s) {
  int v = (s.root == R_K) ? 1 : 0;
  v |= int(s.hops.size()) << 1;
  for (size_t h = 0; h < s.hops.size(); ++h) v |= s.hops[h] << (3 + 4 * h);
  return v;
}

int enc_base(const Base& b, int64_t coef) {
  int kind = 0, arg = 0;
  switch (b.kind) {
    case K_IDX: kind = BK_IDX; break;
    case K_N: kind = BK_N; break;
    case K_SCALAR: kind = BK_SCALAR; arg = b.arg; break;
    case K_START: kind = BK_START; arg = enc_sel(b.sel); break;
    case K_END: kind = BK_END; arg = enc_sel(b.sel); break;
    case K_SEGID: kind = BK_SEGID; arg = enc_sel(b.sel); break;
    default: throw SpecError("internal: free variable in a term");
  }
  if (arg > 0xFFF) throw SpecError("parameter index too large");
  return kind | (coef < 0 ? 8 : 0) | (arg << 4);
}

struct Enc {
  std::vector<int32_t> w;
  void term(const Lin& l) {
    int b[2] = {0, 0}, n = 0;
    for (auto& kv : l.c) b[n++] = enc_base(kv.first, kv.second);
    w.push_back(b[0] | (b[1] << 16));
    w.push_back(int32_t(l.k));
  }
  void atom(const Cond& c) {
    int op = c.op == LT ? OP_LT : c.op == LE ? OP_LE : c.op == EQ ? OP_EQ : OP_NE;
    w.push_back(op);
    term(c.lin);
  }
};

// ---------------------------------------------------------------- listing

std::string sel_str(const Sel& s, const std::string& idx) {
  std::string r = s.root == R_K ? "k" : ("seg(" + idx + ")");
  for (int h : s.hops) r = "ref(" + r + "," + std::to_string(h) + ")";
  return r;
}

std::string lin_str(const Lin& l, const std::string& idx, const std::vector<std::string>& params) {
  std::ostringstream o;
  bool first = true;
  for (auto& kv : l.c) {
    const Base& b = kv.first;
    std::string name;
    switch (b.kind) {
      case K_IDX: name = idx; break;
      case K_N: name = "N"; break;
      case K_SCALAR: name = params[b.arg]; break;
      case K_START: name = "start(" + sel_str(b.sel, idx) + ")"; break;
      case K_END: name = "end(" + sel_str(b.sel, idx) + ")"; break;
      case K_SEGID: name = sel_str(b.sel, idx); break;
      default: name = "?";
    }
    if (kv.second < 0) o << (first ? "-" : " - ");
    else if (!first) o << " + ";
    o << name;
    first = false;
  }
  if (first) o << l.k;
  else if (l.k > 0) o << " + " << l.k;
  else if (l.k < 0) o << " - " << -l.k;
  return o.str();
}

std::string cond_str(const Cond& c, const std::string& idx, const std::vector<std::string>& params) {
  const char* op = c.op == LT ? "<" : c.op == LE ? "<=" : c.op == EQ ? "==" : "!=";
  return lin_str(c.lin, idx, params) + " " + op + " 0";
}

}  // namespace

// ---------------------------------------------------------------- entry

static std::atomic<uint64_t> g_spec_ids{1};

cm_status compile_spec(const char* text, cm_spec** out) {
  try {
    Parser ps;
    ps.t = lex(text);
    std::vector<RegionAst> regions[2];
    int dir = -1;
    bool seen[2] = {false, false};
    while (ps.cur().kind != Tok::END) {
      if (ps.cur().kind != Tok::ID || !is_stmt_keyword(ps.cur().s)) ps.err("expected a statement keyword");
      std::string kw = ps.t[ps.p++].s;
      if (kw == "mask") {
        ps.expect_id();
      } else if (kw == "param") {
        if (dir >= 0) ps.err("param must come before forward/backward");
        do {
          std::string n = ps.expect_id();
          if (n == "i" || n == "j" || n == "N" || n == "k") ps.err("reserved parameter name");
          if (std::find(ps.params.begin(), ps.params.end(), n) != ps.params.end()) ps.err("duplicate parameter");
          ps.params.push_back(n);
        } while (ps.is_op(",") && (++ps.p, true));
      } else if (kw == "refs") {
        if (dir >= 0) ps.err("refs must come before forward/backward");
        int64_t r = ps.expect_num();
        if (r > kMaxRefs) ps.err("too many references per segment");
        ps.n_refs = int(r);
      } else if (kw == "forward" || kw == "backward") {
        dir = (kw == "forward") ? 0 : 1;
        if (seen[dir]) ps.err("section given twice");
        seen[dir] = true;
      } else {  // region
        if (dir < 0) ps.err("region before forward/backward");
        ps.idx_var = dir == 0 ? "i" : "j";
        ps.free_var = dir == 0 ? "j" : "i";
        RegionAst r;
        r.line = ps.cur().line;
        r.name = ps.expect_id();
        ps.expect_op(":");
        r.guard = ps.parse_or();
        ps.expect_op("=>");
        r.rule = ps.parse_or();
        if (!(ps.cur().kind == Tok::END || (ps.cur().kind == Tok::ID && is_stmt_keyword(ps.cur().s))))
          ps.err("unexpected text after the rule");
        regions[dir].push_back(std::move(r));
      }
    }
    if (!seen[0] || !seen[1]) throw SpecError("a spec needs a forward and a backward section");

    std::unique_ptr<cm_spec> sp(new cm_spec());
    sp->params = ps.params;
    sp->n_refs = ps.n_refs;
    std::ostringstream listing;
    Enc enc;
    enc.w = {0, 0};
    for (int d = 0; d < 2; ++d) {
      const std::string idx = d == 0 ? "i" : "j", fr = d == 0 ? "j" : "i";
      std::vector<RegionIR> irs;
      for (auto& ra : regions[d]) {
        BP g = nnf(std::move(ra.guard), false);
        BP r = nnf(std::move(ra.rule), false);
        DNF gd, rd;
        try {
          gd = to_dnf(g.get(), false);
          rd = to_dnf(r.get(), true);
        } catch (const SpecError& e) {
          throw SpecError("line " + std::to_string(ra.line) + " (region " + ra.name + "): " + e.what());
        }
        for (auto& gc : gd) {
          if (gc.family || !gc.lo.empty() || !gc.hi.empty())
            throw SpecError("line " + std::to_string(ra.line) + ": a guard may only test the index");
          // guard DNF: every conjunction becomes its own Region with the same rule
          std::vector<std::vector<Cond>> alts = gc.conds.empty() ? std::vector<std::vector<Cond>>{{}} : gc.conds;
          for (auto& alt : alts) {
            RegionIR ir;
            ir.name = ra.name;
            for (auto& c : alt) {
              for (auto& kv : c.lin.c)
                if ((kv.first.kind == K_START || kv.first.kind == K_END || kv.first.kind == K_SEGID) &&
                    kv.first.sel.root == R_K)
                  throw SpecError("line " + std::to_string(ra.line) + ": guard uses an exists variable");
              int v = const_cond(c);
              if (v == 1) continue;
              ir.guard.push_back(c);
            }
            if (std::any_of(alt.begin(), alt.end(), [](const Cond& c) { return const_cond(c) == 0; })) continue;
            ir.slots = rd;
            Prover pv;
            pv.build(ir.guard, ir.slots);
            for (int it = 0; it < 16 && canonicalise_once(ir.slots, pv); ++it) {
              pv.build(ir.guard, ir.slots);
            }
            irs.push_back(std::move(ir));
          }
        }
      }
      if (irs.size() > size_t(kMaxRegions)) throw SpecError("too many regions");
      sp->dir_off[d] = int(enc.w.size());
      enc.w.push_back(int32_t(irs.size()));
      listing << (d == 0 ? "forward" : "backward") << " (index " << idx << ", free " << fr << ")\n";
      for (auto& ir : irs) {
        if (ir.guard.size() > 255 || ir.slots.size() > 255) throw SpecError("region too large");
        enc.w.push_back(int32_t(ir.guard.size() | (ir.slots.size() << 8)));
        for (auto& c : ir.guard) enc.atom(c);
        int plain = 0, fam = 0;
        listing << "  region " << ir.name << " when";
        if (ir.guard.empty()) listing << " true";
        for (size_t a = 0; a < ir.guard.size(); ++a)
          listing << (a ? " & " : " ") << cond_str(ir.guard[a], idx, sp->params);
        listing << "\n";
        for (auto& s : ir.slots) {
          if (s.lo.size() > 15 || s.hi.size() > 15 || s.conds.size() > 15) throw SpecError("slot too large");
          (s.family ? fam : plain) += 1;
          enc.w.push_back(int32_t((s.family ? 1 : 0) | (s.lo.size() << 4) | (s.hi.size() << 8) | (s.conds.size() << 12)));
          for (auto& l : s.lo) enc.term(l);
          for (auto& l : s.hi) enc.term(l);
          for (auto& cj : s.conds) {
            enc.w.push_back(int32_t(cj.size()));
            for (auto& c : cj) enc.atom(c);
          }
          listing << "    slot" << (s.family ? " exists k:" : "") << " " << fr << " in [";
          if (s.lo.empty()) listing << "0";
          else if (s.lo.size() == 1) listing << lin_str(s.lo[0], idx, sp->params);
          else {
            listing << "max(";
            for (size_t a = 0; a < s.lo.size(); ++a) listing << (a ? ", " : "") << lin_str(s.lo[a], idx, sp->params);
            listing << ")";
          }
          listing << ", ";
          if (s.hi.empty()) listing << "N";
          else if (s.hi.size() == 1) listing << lin_str(s.hi[0], idx, sp->params);
          else {
            listing << "min(";
            for (size_t a = 0; a < s.hi.size(); ++a) listing << (a ? ", " : "") << lin_str(s.hi[a], idx, sp->params);
            listing << ")";
          }
          listing << ")";
          if (!s.conds.empty()) {
            listing << " if ";
            for (size_t a = 0; a < s.conds.size(); ++a) {
              listing << (a ? " | (" : "(");
              for (size_t b = 0; b < s.conds[a].size(); ++b)
                listing << (b ? " & " : "") << cond_str(s.conds[a][b], idx, sp->params);
              listing << ")";
            }
          }
          listing << "\n";
        }
        sp->region_slots[d].push_back({plain, fam});
      }
    }
    enc.w[0] = int32_t(enc.w.size());
    enc.w[1] = sp->dir_off[1];
    if (enc.w.size() > size_t(kProgMaxWords))
      throw SpecError("lowered program needs " + std::to_string(enc.w.size()) + " words > " +
                      std::to_string(kProgMaxWords));
    for (size_t i = 0; i < size_t(kProgMaxWords); ++i) sp->prog.w[i] = i < enc.w.size() ? enc.w[i] : 0;
    sp->n_words = int(enc.w.size());
    sp->listing = listing.str();
    sp->id = g_spec_ids.fetch_add(1);
    *out = sp.release();
    return CM_OK;
  } catch (const SpecError& e) {
    return fail(CM_ERR_PARSE, e.what());
  } catch (const std::exception& e) {
    return fail(CM_ERR_PARSE, std::string("spec compiler: ") + e.what());
  }
}

int spec_width(const cm_spec* spec, int dir, int seg_cap) {
  int k = 1;
  for (auto& rs : spec->region_slots[dir]) k = std::max(k, rs.first + rs.second * seg_cap);
  return k;
}

}  // namespace cm
