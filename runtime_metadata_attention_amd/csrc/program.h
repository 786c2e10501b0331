// program.h -- encoding and evaluation of a lowered MaskSpec (endpoint program).
//
// The symbolic compiler (spec.cpp) lowers each Region's visibility rule to a
// list of interval slots (CompileMask paper summary, section 3.2.2 "Symbolic
// Lowering to Visible Intervals").  This header fixes the flat int32 encoding
// of that result and the routine that evaluates it for one index against one
// sample's metadata (section 3.3 "Online Efficient Mask Attention Execution":
// the preprocess kernel evaluates the compiled endpoints).  The same code runs
// in the preprocess kernel and in the host inspection entry point.
//
// Encoding (all int32):
//   program   : [0] total words, [1] word offset of the backward direction;
//               the forward direction starts at word 2
//   direction : n_regions, then the regions
//   region    : n_guard_atoms | n_slots << 8, guard atoms, slots
//   slot      : flags (bit 0 = exists-slot) | n_lo << 4 | n_hi << 8 | n_conj << 12,
//               n_lo terms, n_hi terms, n_conj conjunctions of condition atoms
//               (each: n_atoms, then the atoms)
//   atom      : op, term      meaning  term <op> 0, op in {LT, LE, EQ, NE}
//   term      : base0 | base1 << 16, constant  (value = base0 + base1 + constant)
//   base (16b): kind (bits 0-2), negate (bit 3), arg (bits 4-15)
//               SCALAR: arg = scalar index; START/END/SEGID: arg = selector
//   selector  : root (bit 0: 0 = segment holding the index, 1 = the exists
//               variable k), hops (bits 1-2), hop ref index h at bits 3+4h
// A slot's interval is [max(0, lo terms), min(N, hi terms)), empty slots are
// dropped.  An atom or a bound that names a missing segment (-1, a reference
// that is absent) is false.  An index uses the first Region whose guard holds;
// an index in no Region sees nothing.
#pragma once
#ifdef __HIPCC_RTC__
// the run-time compiler keeps the fixed-width types in its own namespace
typedef __hip_internal::int32_t int32_t;
typedef __hip_internal::uint32_t uint32_t;
typedef __hip_internal::int64_t int64_t;
typedef __hip_internal::uint64_t uint64_t;
#else
#include <stdint.h>
#endif

#if defined(__HIPCC_RTC__)
#define CM_HD __host__ __device__ __forceinline__
#elif defined(__HIPCC__) || defined(__HIP__)
#include <hip/hip_runtime.h>
#define CM_HD __host__ __device__ __forceinline__
#else
#define CM_HD inline
#endif

namespace cm {

constexpr int kProgMaxWords = 448;  // kernel-argument budget for both directions
constexpr int kMaxRegions = 16;
constexpr int kMaxRefs = 15;

enum BaseKind : int { BK_NONE = 0, BK_IDX = 1, BK_N = 2, BK_SCALAR = 3, BK_START = 4, BK_END = 5, BK_SEGID = 6 };
enum AtomOp : int { OP_LT = 0, OP_LE = 1, OP_EQ = 2, OP_NE = 3 };

struct Program {
  int32_t w[kProgMaxWords];
};

// One sample's metadata as the evaluator sees it.
struct SampleView {
  int32_t N;
  int32_t n_seg;
  int32_t n_refs;
  const int32_t* scalars;  // [n_scalars]
  const int32_t* bounds;   // [n_seg + 1]
  const int32_t* refs;     // [seg_cap][n_refs]
};

// Segment holding position x: the last t with bounds[t] <= x, if x < bounds[n_seg].
CM_HD int segment_of(const SampleView& s, int x) {
  if (s.n_seg <= 0) return -1;
  if (x < s.bounds[0] || x >= s.bounds[s.n_seg]) return -1;
  int lo = 0, hi = s.n_seg;  // invariant: bounds[lo] <= x < bounds[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (s.bounds[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

CM_HD int resolve_selector(const SampleView& s, int sel, int idx_seg, int k) {
  int g = (sel & 1) ? k : idx_seg;
  const int hops = (sel >> 1) & 3;
  for (int h = 0; h < hops; ++h) {
    if (g < 0 || g >= s.n_seg) return -1;
    const int r = (sel >> (3 + 4 * h)) & 15;
    if (r >= s.n_refs) return -1;
    g = s.refs[g * s.n_refs + r];
  }
  return (g >= 0 && g < s.n_seg) ? g : -1;
}

// Value of one 16-bit base; false when it names a missing segment.
CM_HD bool eval_base(const SampleView& s, int base, int idx, int idx_seg, int k, int64_t& acc) {
  const int kind = base & 7;
  const int arg = (base >> 4) & 0xFFF;
  int64_t v = 0;
  switch (kind) {
    case BK_NONE: return true;
    case BK_IDX: v = idx; break;
    case BK_N: v = s.N; break;
    case BK_SCALAR: v = s.scalars[arg]; break;
    default: {
      const int g = resolve_selector(s, arg, idx_seg, k);
      if (g < 0) return false;
      v = kind == BK_START ? s.bounds[g] : kind == BK_END ? s.bounds[g + 1] : g;
    }
  }
  acc += (base & 8) ? -v : v;
  return true;
}

CM_HD bool eval_term(const SampleView& s, const int32_t* t, int idx, int idx_seg, int k, int64_t& v) {
  v = t[1];
  const int b0 = t[0] & 0xFFFF, b1 = (t[0] >> 16) & 0xFFFF;
  return eval_base(s, b0, idx, idx_seg, k, v) && eval_base(s, b1, idx, idx_seg, k, v);
}

CM_HD bool eval_atom(const SampleView& s, const int32_t* a, int idx, int idx_seg, int k) {
  int64_t v;
  if (!eval_term(s, a + 1, idx, idx_seg, k, v)) return false;
  switch (a[0]) {
    case OP_LT: return v < 0;
    case OP_LE: return v <= 0;
    case OP_EQ: return v == 0;
    default: return v != 0;
  }
}

constexpr int kAtomWords = 3;
constexpr int kTermWords = 2;

// Words of a slot starting at p (depends only on program words: uniform).
CM_HD int slot_words(const int32_t* p) {
  const int hdr = p[0];
  const int n_lo = (hdr >> 4) & 15, n_hi = (hdr >> 8) & 15, n_conj = (hdr >> 12) & 15;
  int w = 1 + kTermWords * (n_lo + n_hi);
  for (int c = 0; c < n_conj; ++c) w += 1 + kAtomWords * p[w];
  return w;
}

// A slot's condition (a disjunction of conjunctions of atoms) for one value
// of the exists variable k; true when the slot has none.
CM_HD bool slot_cond(const SampleView& s, const int32_t* p, int idx, int idx_seg, int k) {
  const int hdr = p[0];
  const int n_lo = (hdr >> 4) & 15, n_hi = (hdr >> 8) & 15, n_conj = (hdr >> 12) & 15;
  if (n_conj == 0) return true;
  const int32_t* q = p + 1 + kTermWords * (n_lo + n_hi);
  bool any = false;
  for (int c = 0; c < n_conj; ++c) {
    const int na = q[0];
    bool all = true;
    for (int a = 0; a < na; ++a) all = all && eval_atom(s, q + 1 + kAtomWords * a, idx, idx_seg, k);
    any = any || all;
    q += 1 + kAtomWords * na;
  }
  return any;
}
// True when no term of the slot (bounds or condition) reads the index itself:
// the slot then depends on the index only through the index's segment.
CM_HD bool slot_index_free(const int32_t* p) {
  const int hdr = p[0];
  const int n_lo = (hdr >> 4) & 15, n_hi = (hdr >> 8) & 15, n_conj = (hdr >> 12) & 15;
  const int32_t* q = p + 1;
  for (int t = 0; t < n_lo + n_hi; ++t, q += kTermWords)
    if ((q[0] & 7) == BK_IDX || ((q[0] >> 16) & 7) == BK_IDX) return false;
  for (int c = 0; c < n_conj; ++c) {
    const int na = q[0];
    for (int a = 0; a < na; ++a) {
      const int32_t* t = q + 1 + kAtomWords * a + 1;
      if ((t[0] & 7) == BK_IDX || ((t[0] >> 16) & 7) == BK_IDX) return false;
    }
    q += 1 + kAtomWords * na;
  }
  return true;
}

// A slot's interval [lo, hi) for one value of the exists variable k, its
// condition aside.  Returns true when the interval is non-empty.
CM_HD bool slot_bounds(const SampleView& s, const int32_t* p, int idx, int idx_seg, int k,
                       int32_t& lo_out, int32_t& hi_out) {
  const int hdr = p[0];
  const int n_lo = (hdr >> 4) & 15, n_hi = (hdr >> 8) & 15;
  const int32_t* q = p + 1;
  int64_t lo = 0, hi = s.N;
  bool ok = true;
  for (int t = 0; t < n_lo; ++t, q += kTermWords) {
    int64_t v;
    ok = ok && eval_term(s, q, idx, idx_seg, k, v);
    if (ok && v > lo) lo = v;
  }
  for (int t = 0; t < n_hi; ++t, q += kTermWords) {
    int64_t v;
    ok = ok && eval_term(s, q, idx, idx_seg, k, v);
    if (ok && v < hi) hi = v;
  }
  if (hi > s.N) hi = s.N;
  if (lo < 0) lo = 0;
  lo_out = (int32_t)lo;
  hi_out = (int32_t)hi;
  return ok && lo < hi;
}

// Evaluate a slot for one value of the exists variable k.  Returns true and
// [lo, hi) when the slot contributes a non-empty interval.  The condition
// comes first: for most k an exists-slot's condition is false, and then its
// bounds need not be evaluated.
CM_HD bool eval_slot(const SampleView& s, const int32_t* p, int idx, int idx_seg, int k,
                     int32_t& lo_out, int32_t& hi_out) {
  return slot_cond(s, p, idx, idx_seg, k) && slot_bounds(s, p, idx, idx_seg, k, lo_out, hi_out);
}

#if defined(__HIP_DEVICE_COMPILE__)
// An exists-slot evaluated by the whole wave at once.  Each program word
// read is a dependent scalar load, so the per-index loop over every k costs
// a few hundred cycles per k.  When the slot does not read the index itself
// and every active lane's index belongs to the same sample, the slot's
// intervals depend on the lane only through its segment.  The wave then
// takes the distinct segments of its lanes in turn: the active lane of rank
// r (r-th active lane by lane id) evaluates the condition for
// k = k0 + r, a ballot collects the k that hold, every lane evaluates the
// bounds of just those (the same values on every lane), and the lanes of
// that segment emit them, in ascending k as the per-index loop does.
// Returns false (nothing emitted) when the wave does not qualify; the
// caller then loops over k per index.
template <class Emit>
__device__ __forceinline__ bool exists_by_wave(const SampleView& s, const int32_t* p, int idx, int idx_seg,
                                               Emit&& emit) {
  if (!slot_index_free(p)) return false;  // program words: wave-uniform
  const uint64_t active = __builtin_amdgcn_ballot_w64(true);
  const uint64_t bp = (uint64_t)(const void*)s.bounds;
  const uint32_t b_lo = __builtin_amdgcn_readfirstlane(uint32_t(bp)), b_hi = __builtin_amdgcn_readfirstlane(uint32_t(bp >> 32));
  if (__builtin_amdgcn_ballot_w64(uint32_t(bp) == b_lo && uint32_t(bp >> 32) == b_hi) != active) return false;
  // inactive lanes take no k: ranks count active lanes only
  const int rank = int(__builtin_amdgcn_mbcnt_hi(uint32_t(active >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(active), 0u)));
  const int n_active = __builtin_popcountll(active);
  uint64_t todo = active;
  while (todo != 0) {
    const int leader = __builtin_ctzll(todo);
    const int seg0 = __builtin_amdgcn_readlane(idx_seg, leader);
    const bool mine = idx_seg == seg0;
    todo &= ~__builtin_amdgcn_ballot_w64(mine);
    for (int k0 = 0; k0 < s.n_seg; k0 += n_active) {
      const int k = k0 + rank;
      const bool c = k < s.n_seg && slot_cond(s, p, idx, seg0, k);
      uint64_t m = __builtin_amdgcn_ballot_w64(c);
      while (m != 0) {
        const int lane = __builtin_ctzll(m);
        const int kk = k0 + __builtin_popcountll(active & ((uint64_t(1) << lane) - 1));
        m &= m - 1;
        int32_t lo, hi;
        if (slot_bounds(s, p, idx, seg0, kk, lo, hi) && mine) emit(lo, hi);
      }
    }
  }
  return true;
}
#endif

// Walk one direction's regions for index idx and hand every non-empty slot
// interval to emit(lo, hi).  Program words are read at offsets that depend
// only on the program, so on the GPU every read is wave-uniform.
template <class Emit>
CM_HD void eval_direction(const int32_t* prog, int dir_off, const SampleView& s, int idx, Emit&& emit) {
  const int32_t* p = prog + dir_off;
  const int n_regions = p[0];
  ++p;
  const int idx_seg = segment_of(s, idx);
  bool matched = false;
  for (int r = 0; r < n_regions; ++r) {
    const int n_guard = p[0] & 255, n_slots = (p[0] >> 8) & 255;
    ++p;
    bool g = !matched;
    for (int a = 0; a < n_guard; ++a) g = g && eval_atom(s, p + kAtomWords * a, idx, idx_seg, -1);
    p += kAtomWords * n_guard;
    for (int sl = 0; sl < n_slots; ++sl) {
      if (g) {
        if (p[0] & 1) {
          bool done = false;
#if defined(__HIP_DEVICE_COMPILE__)
          done = exists_by_wave(s, p, idx, idx_seg, emit);
#endif
          for (int k = 0; !done && k < s.n_seg; ++k) {
            int32_t lo, hi;
            if (eval_slot(s, p, idx, idx_seg, k, lo, hi)) emit(lo, hi);
          }
        } else {
          int32_t lo, hi;
          if (eval_slot(s, p, idx, idx_seg, -1, lo, hi)) emit(lo, hi);
        }
      }
      p += slot_words(p);
    }
    matched = matched || g;
  }
}

// Metadata validity of one sample (the CM_MD_* bits).
CM_HD uint32_t validate_sample(int32_t N, int32_t n_seg, int32_t seg_cap, const int32_t* bounds,
                               const int32_t* refs, int32_t n_refs) {
  if (n_seg < 0 || n_seg > seg_cap) return 1u;
  uint32_t err = 0;
  if (n_seg >= 1) {
    for (int t = 0; t <= n_seg; ++t) {
      if (bounds[t] < 0 || bounds[t] > N) err |= 4u;
      if (t < n_seg && bounds[t + 1] < bounds[t]) err |= 2u;
    }
    for (int t = 0; t < n_seg * n_refs; ++t)
      if (refs[t] < -1 || refs[t] >= n_seg) err |= 8u;
  }
  return err;
}

}  // namespace cm
