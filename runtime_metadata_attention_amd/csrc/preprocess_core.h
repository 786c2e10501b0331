// preprocess_core.h -- the preprocess kernel's device code (batch metadata ->
// Execution Descriptor), shared by two instantiations:
//   * preprocess.hip: the lowered program read from the kernel arguments and
//     interpreted (every spec, no compile step);
//   * a spec-specialised kernel compiled at run time (cm_spec_specialize):
//     the same code with the program as a compile-time constant array, which
//     the compiler folds into straight-line endpoint arithmetic.
// See preprocess.hip for what the kernel computes.  This header is
// self-contained (HIP device code, program.h and preprocess_args.h) so that
// the run-time compiler can take it as is.
#pragma once
#include "preprocess_args.h"
#include "program.h"

namespace cm {
namespace pre {

constexpr int kThreads = kPreThreads;

struct Role {
  int x0, nidx;          // first index and index count of this tile
  int K;                 // table width
  uint2* table;          // this sample's interval table
  int Bt, T, W;          // tile width / count / words along the other axis
  uint32_t* bitmap;      // this tile's bitmap row
  uint32_t* tkmax;       // this tile's run maximum
  int dir_off;
};

struct Lds {
  int32_t* any;
  int32_t* full;
  int32_t* misc;         // [0] run max, [1] sample error, [2] error OR over samples, [3] cu_seqlens error
};

__device__ __forceinline__ void count_run(const Lds& L, const Role& r, int N, uint32_t s, uint32_t e) {
  const int a0 = int(s) / r.Bt, a1 = int(e - 1) / r.Bt;
  atomicAdd(&L.any[a0], 1);
  atomicAdd(&L.any[a1 + 1], -1);
  const int f0 = (int(s) + r.Bt - 1) / r.Bt;
  const int f1 = (int(e) == N) ? r.T : int(e) / r.Bt;
  if (f0 < f1) {
    atomicAdd(&L.full[f0], 1);
    atomicAdd(&L.full[f1], -1);
  }
}

// Where an index's rule is evaluated: the sample's metadata, the index in the
// sample's coordinates, and the shift from those to the descriptor's (0 for a
// padded batch; the sample's first token for a packed one).
struct Site {
  SampleView sv;
  int local;       // index inside the sample
  int global;      // index in the descriptor (its table row)
  uint32_t shift;  // added to the evaluated endpoints
};

// Runs held in registers: sorted insertion with compile-time indices only.
template <int KC>
__device__ __forceinline__ void runs_registers(const int32_t* prog, const Site& st, const Role& r, const Lds& L, int N) {
  uint32_t s[KC], e[KC];
  int n = 0;
#pragma unroll
  for (int q = 0; q < KC; ++q) { s[q] = 0; e[q] = 0; }
  eval_direction(prog, r.dir_off, st.sv, st.local, [&](int32_t lo_, int32_t hi_) {
    const uint32_t lo = uint32_t(lo_) + st.shift, hi = uint32_t(hi_) + st.shift;
    int pos = 0;
#pragma unroll
    for (int q = 0; q < KC; ++q) pos += (q < n && s[q] <= lo) ? 1 : 0;
#pragma unroll
    for (int q = KC - 1; q >= 0; --q) {
      if (q > 0 && q > pos && q <= n) { s[q] = s[q - 1]; e[q] = e[q - 1]; }
      else if (q == pos) { s[q] = lo; e[q] = hi; }
    }
    n = n < KC ? n + 1 : KC;
  });
  uint2* row = r.table + size_t(st.global) * r.K;
  int nout = 0;
  uint32_t cs = 0, ce = 0;
  bool open = false;
#pragma unroll
  for (int q = 0; q < KC; ++q) {
    if (q < n) {
      if (open && s[q] <= ce) {
        ce = e[q] > ce ? e[q] : ce;
      } else {
        if (open) { row[nout++] = make_uint2(cs, ce); count_run(L, r, N, cs, ce); }
        cs = s[q]; ce = e[q]; open = true;
      }
    }
  }
  if (open) { row[nout++] = make_uint2(cs, ce); count_run(L, r, N, cs, ce); }
  for (int q = nout; q < r.K; ++q) row[q] = make_uint2(0u, 0u);
  atomicMax(&L.misc[0], nout);
}

// Wide tables (exists-slots): sort and merge in the index's own table row.
__device__ __forceinline__ void runs_memory(const int32_t* prog, const Site& st, const Role& r, const Lds& L, int N) {
  uint2* row = r.table + size_t(st.global) * r.K;
  int n = 0;
  const int K = r.K;
  eval_direction(prog, r.dir_off, st.sv, st.local, [&](int32_t lo_, int32_t hi_) {
    if (n >= K) return;
    const uint32_t lo = uint32_t(lo_) + st.shift, hi = uint32_t(hi_) + st.shift;
    int pos = n;
    while (pos > 0 && row[pos - 1].x > lo) { row[pos] = row[pos - 1]; --pos; }
    row[pos] = make_uint2(lo, hi);
    ++n;
  });
  int nout = 0;
  uint32_t cs = 0, ce = 0;
  bool open = false;
  for (int q = 0; q < n; ++q) {
    const uint2 v = row[q];
    if (open && v.x <= ce) {
      ce = v.y > ce ? v.y : ce;
    } else {
      if (open) { row[nout++] = make_uint2(cs, ce); count_run(L, r, N, cs, ce); }
      cs = v.x; ce = v.y; open = true;
    }
  }
  if (open) { row[nout++] = make_uint2(cs, ce); count_run(L, r, N, cs, ce); }
  // the rest of the row was cleared by the work-group (wide_table_clear);
  // only the entries the sort used past the merged runs are stale
  for (int q = nout; q < n; ++q) row[q] = make_uint2(0u, 0u);
  atomicMax(&L.misc[0], nout);
}

// An index of an invalid sample sees nothing: an all-zero row (wide rows
// were cleared already).
__device__ __forceinline__ void clear_row(const Role& r, int idx) {
  if (r.K > 8) return;
  uint2* row = r.table + size_t(idx) * r.K;
  for (int t = 0; t < r.K; ++t) row[t] = make_uint2(0u, 0u);
}

// The runs of one index, by table width.
__device__ __forceinline__ void build_runs(const int32_t* prog, const Site& st, const Role& r, const Lds& L, int N) {
  if (r.K <= 1) runs_registers<1>(prog, st, r, L, N);
  else if (r.K <= 2) runs_registers<2>(prog, st, r, L, N);
  else if (r.K <= 4) runs_registers<4>(prog, st, r, L, N);
  else if (r.K <= 8) runs_registers<8>(prog, st, r, L, N);
  else runs_memory(prog, st, r, L, N);
}

// Clear the work-group's rows of a wide table (more than 8 entries per
// index) with coalesced stores: the rows of consecutive indices are one
// contiguous block.  Each index then writes only its runs.
__device__ __forceinline__ void wide_table_clear(const Role& r) {
  uint2* block = r.table + size_t(r.x0) * r.K;
  const int total = r.nidx * r.K;
  for (int t = threadIdx.x; t < total; t += kThreads) block[t] = make_uint2(0u, 0u);
}

// In-place inclusive prefix sums of a[0..T) and b[0..T) by one work-group:
// each thread sums a contiguous chunk, the chunk sums are scanned within each
// wave by shuffles and across the waves through `part`, and each thread then
// rewrites its chunk as running sums.  Two barriers.
__device__ void scan2(int32_t* a, int32_t* b, int T, int32_t* part) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int chunk = (T + kThreads - 1) / kThreads;
  const int lo = t * chunk, hi = min(T, lo + chunk);
  int32_t ca = 0, cb = 0;
  for (int c = lo; c < hi; ++c) { ca += a[c]; cb += b[c]; }
  int32_t sa = ca, sb = cb;  // inclusive scan of the chunk sums within the wave
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t xa = __shfl_up(sa, off, 64), xb = __shfl_up(sb, off, 64);
    if (lane >= off) { sa += xa; sb += xb; }
  }
  if (lane == 63) { part[wv] = sa; part[kThreads + wv] = sb; }
  __syncthreads();
  int32_t ra = sa - ca, rb = sb - cb;  // exclusive: the chunks before this one
  for (int w = 0; w < wv; ++w) { ra += part[w]; rb += part[kThreads + w]; }
  for (int c = lo; c < hi; ++c) {
    ra += a[c]; a[c] = ra;
    rb += b[c]; b[c] = rb;
  }
  __syncthreads();
}

// Bits 0..15 of x moved to the even bit positions 0, 2, .., 30.
__device__ __forceinline__ uint32_t spread16(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  x = (x | (x << 1)) & 0x55555555u;
  return x;
}

// Metadata checks of one padded sample (the CM_MD_* bits validate_sample
// forms), spread over the work-group and OR-ed into *err.
__device__ __forceinline__ void validate_sample_wg(int32_t N, int32_t n_seg, int32_t seg_cap, const int32_t* bounds,
                                                   const int32_t* refs, int32_t n_refs, int32_t* err) {
  const int t = threadIdx.x;
  uint32_t e = 0;
  if (n_seg < 0 || n_seg > seg_cap) {
    e = t == 0 ? 1u : 0u;
  } else if (n_seg >= 1) {
    for (int i = t; i <= n_seg; i += kThreads) {
      if (bounds[i] < 0 || bounds[i] > N) e |= 4u;
      if (i < n_seg && bounds[i + 1] < bounds[i]) e |= 2u;
    }
    for (int i = t; i < n_seg * n_refs; i += kThreads)
      if (refs[i] < -1 || refs[i] >= n_seg) e |= 8u;
  }
  if (e != 0) atomicOr(reinterpret_cast<uint32_t*>(err), e);
}

// The kernel body for one work-group; `prog` is the lowered program (both
// directions).  Grid (Tq_f + Tk_b, B), kThreads threads, dynamic LDS of
// preprocess_lds_words(a) words.
__device__ __forceinline__ void preprocess_body(const PreprocessArgs& a, const int32_t* prog) {
  extern __shared__ int32_t lds[];
  const int b = blockIdx.y;
  const bool row_role = int(blockIdx.x) < a.Tq_f;
  const int tile = row_role ? int(blockIdx.x) : int(blockIdx.x) - a.Tq_f;
  uint32_t* desc = a.desc;

  Role r;
  if (row_role) {
    r.x0 = tile * a.fq; r.nidx = min(a.fq, a.N - r.x0); r.K = a.K_r;
    r.table = reinterpret_cast<uint2*>(desc + a.off_words[SEC_ROW_IV]) + size_t(b) * a.N * a.K_r;
    r.Bt = a.fk; r.T = a.Tk_f; r.W = a.Wf;
    r.bitmap = desc + a.off_words[SEC_FBM] + (size_t(b) * a.Tq_f + tile) * a.Wf;
    r.tkmax = desc + a.off_words[SEC_ROW_TKMAX] + size_t(b) * a.Tq_f + tile;
    r.dir_off = a.dir_off[0];
  } else {
    r.x0 = tile * a.bk; r.nidx = min(a.bk, a.N - r.x0); r.K = a.K_c;
    r.table = reinterpret_cast<uint2*>(desc + a.off_words[SEC_COL_IV]) + size_t(b) * a.N * a.K_c;
    r.Bt = a.bq; r.T = a.Tq_b; r.W = a.Wb;
    r.bitmap = desc + a.off_words[SEC_BBM] + (size_t(b) * a.Tk_b + tile) * a.Wb;
    r.tkmax = desc + a.off_words[SEC_COL_TKMAX] + size_t(b) * a.Tk_b + tile;
    r.dir_off = a.dir_off[1];
  }

  // LDS: any[Tmax+1] full[Tmax+1] part[2*threads] misc[4] bounds[seg_cap+1] refs[..] scalars[..]
  const int Tmax = max(a.Tk_f, a.Tq_b);
  Lds L;
  L.any = lds;
  L.full = lds + (Tmax + 1);
  int32_t* part = L.full + (Tmax + 1);
  L.misc = part + 2 * kThreads;
  int32_t* bounds = L.misc + 4;
  int32_t* refs = bounds + (a.seg_cap + 1);
  int32_t* scal = refs + a.seg_cap * a.n_refs;

  const int tid = threadIdx.x;
  const bool packed = a.cu_seqlens != nullptr;
  const int n_meta = packed ? a.n_samples : a.B;  // metadata rows
  // a padded batch caches sample b's metadata in LDS; a packed batch reads
  // each index's sample from global memory
  const int n_seg = (!packed && a.n_seg) ? a.n_seg[b] : 0;
  if (!packed) {
    for (int t = tid; t <= a.seg_cap && a.seg_bounds; t += kThreads) bounds[t] = a.seg_bounds[size_t(b) * (a.seg_cap + 1) + t];
    for (int t = tid; t < a.seg_cap * a.n_refs; t += kThreads) refs[t] = a.refs[size_t(b) * a.seg_cap * a.n_refs + t];
    for (int t = tid; t < a.n_scalars; t += kThreads) scal[t] = a.scalars[size_t(b) * a.n_scalars + t];
  }
  for (int t = tid; t <= r.T; t += kThreads) { L.any[t] = 0; L.full[t] = 0; }
  if (tid == 0) { L.misc[0] = 0; L.misc[1] = 0; L.misc[2] = 0; L.misc[3] = 0; }
  if (r.K > 8) wide_table_clear(r);  // ordered before the runs by the barriers below
  __syncthreads();
  if (packed) {
    // cu_seqlens must run from 0 to N without decreasing
    for (int t = tid; t <= a.n_samples; t += kThreads) {
      const int c = a.cu_seqlens[t];
      const bool bad = (t == 0 && c != 0) || (t == a.n_samples && c != a.N) ||
                       (t < a.n_samples && a.cu_seqlens[t + 1] < c) || c < 0 || c > a.N;
      if (bad) atomicOr(reinterpret_cast<uint32_t*>(&L.misc[3]), kMdCuSeqlens);
    }
  } else {
    validate_sample_wg(a.N, n_seg, a.seg_cap, bounds, refs, a.n_refs, &L.misc[1]);
  }
  __syncthreads();
  const uint32_t cu_err = uint32_t(L.misc[3]);
  // work-group 0 (of sample 0) forms the error word of every sample; a padded
  // batch's work-groups (0, b) also write sample_err[b] below
  if (blockIdx.x == 0 && b == 0) {
    for (int bb = tid; bb < n_meta; bb += kThreads) {
      const int ns = a.n_seg ? a.n_seg[bb] : 0;
      const int32_t* gb = a.seg_bounds ? a.seg_bounds + size_t(bb) * (a.seg_cap + 1) : nullptr;
      const int32_t* gr = a.refs ? a.refs + size_t(bb) * a.seg_cap * a.n_refs : nullptr;
      uint32_t e;
      if (packed && cu_err) {
        e = cu_err;  // no sample boundaries to check against: every row is empty
      } else {
        const int nlen = packed ? a.cu_seqlens[bb + 1] - a.cu_seqlens[bb] : a.N;
        e = validate_sample(nlen, ns, a.seg_cap, gb, gr, a.n_refs);
      }
      if (packed) desc[a.off_words[SEC_SAMPLE_ERR] + bb] = e;
      atomicOr(reinterpret_cast<uint32_t*>(&L.misc[2]), e);
    }
  }
  __syncthreads();
  const uint32_t err = uint32_t(L.misc[1]);

  for (int q = tid; q < r.nidx; q += kThreads) {
    const int idx = r.x0 + q;
    // The runs are built in two branches with their own views, so that in
    // the padded one the metadata pointers are known to be LDS (ds_read
    // rather than flat loads, which cost several times more in the loops
    // over segments).
    if (!packed) {
      if (err != 0) {
        clear_row(r, idx);
        continue;
      }
      Site st;
      st.global = idx;
      st.sv.N = a.N; st.sv.n_seg = n_seg; st.sv.n_refs = a.n_refs;
      st.sv.scalars = scal; st.sv.bounds = bounds; st.sv.refs = refs;
      st.local = idx;
      st.shift = 0;
      build_runs(prog, st, r, L, a.N);
    } else {
      if (cu_err != 0) {
        clear_row(r, idx);
        continue;
      }
      // the sample holding idx: the last one whose first token is <= idx
      int lo = 0, hi = a.n_samples - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_seqlens[mid] <= idx) lo = mid; else hi = mid - 1;
      }
      const int sb = lo, c0 = a.cu_seqlens[sb];
      const int ns = a.n_seg ? a.n_seg[sb] : 0;
      Site st;
      st.global = idx;
      st.sv.N = a.cu_seqlens[sb + 1] - c0;
      st.sv.n_seg = ns; st.sv.n_refs = a.n_refs;
      st.sv.scalars = a.scalars ? a.scalars + size_t(sb) * a.n_scalars : nullptr;
      st.sv.bounds = a.seg_bounds ? a.seg_bounds + size_t(sb) * (a.seg_cap + 1) : nullptr;
      st.sv.refs = a.refs ? a.refs + size_t(sb) * a.seg_cap * a.n_refs : nullptr;
      st.local = idx - c0;
      st.shift = uint32_t(c0);
      if (validate_sample(st.sv.N, ns, a.seg_cap, st.sv.bounds, st.sv.refs, a.n_refs) != 0) {
        clear_row(r, idx);
        continue;
      }
      build_runs(prog, st, r, L, a.N);
    }
  }
  __syncthreads();
  scan2(L.any, L.full, r.T, part);

  // tile codes (0 empty, 1 full, 2 partial), one tile per thread; each wave's
  // 64 codes become four bitmap words from two ballots
  for (int c0 = 0; c0 < r.T; c0 += kThreads) {
    const int c = c0 + tid;
    uint32_t code = 0;
    if (c < r.T) code = L.any[c] == 0 ? 0u : (L.full[c] == r.nidx ? 1u : 2u);
    const uint64_t lo = __ballot(int(code & 1u)), hi = __ballot(int(code >> 1));
    const int lane = tid & 63;
    const int w = (c0 + (tid & ~63)) / 16 + lane;
    if (lane < 4 && w < r.W) {
      const uint32_t l16 = uint32_t(lo >> (16 * lane)) & 0xFFFFu, h16 = uint32_t(hi >> (16 * lane)) & 0xFFFFu;
      r.bitmap[w] = spread16(l16) | (spread16(h16) << 1);
    }
  }
  if (tid == 0) {
    *r.tkmax = uint32_t(L.misc[0]);
    if (blockIdx.x == 0 && !packed) desc[a.off_words[SEC_SAMPLE_ERR] + b] = err;
    if (blockIdx.x == 0 && b == 0) {
      uint4* h = reinterpret_cast<uint4*>(desc + a.off_words[SEC_HEADER]);
      h[0] = make_uint4(kDescMagic, uint32_t(a.B), uint32_t(a.N), uint32_t(a.K_r));
      h[1] = make_uint4(uint32_t(a.K_c), uint32_t(a.fq), uint32_t(a.fk), uint32_t(a.bk));
      h[2] = make_uint4(uint32_t(a.bq), uint32_t(a.Tq_f), uint32_t(a.Tk_f), uint32_t(a.Tk_b));
      h[3] = make_uint4(uint32_t(a.Tq_b), uint32_t(L.misc[2]), uint32_t(a.seg_cap), uint32_t(a.n_samples));
    }
  }
}

}  // namespace pre
}  // namespace cm
