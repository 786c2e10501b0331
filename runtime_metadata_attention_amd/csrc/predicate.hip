// predicate.hip -- the predicate baseline's block mask (FlexAttention-style).
//
// The CompileMask paper summary (sections 1, 2.1 and 4.2) measures against
// masking that is written as a predicate of (row, key): a block mask is built
// by evaluating the predicate at every element, and the attention kernel
// evaluates it again at every element of a partial tile.  Rebuilding that
// block mask whenever the batch metadata change is the cost the Execution
// Descriptor avoids.  This file builds it, so that both ways can be measured
// on the same kernels:
//   1. tok_seg_kernel: the segment of every token (-1 = none), written into
//      the descriptor's row_iv section as int32 [B][N];
//   2. blockmask_kernel: grid (Tq_f + Tk_b, B) like the preprocess; a
//      work-group owns one forward query tile (or backward key tile), counts
//      the visible elements of its tile row against every tile of the other
//      axis by evaluating the predicate at each of them, and writes the
//      tile codes (0 empty, 1 full, 2 partial), the sample's metadata error
//      word and the header.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "internal.h"

namespace cm {
namespace {

using namespace attn;

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void tok_seg_kernel(PreprocessArgs a) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= int64_t(a.B) * a.N) return;
  const int b = int(t / a.N), x = int(t % a.N);
  int32_t* out = reinterpret_cast<int32_t*>(a.desc + a.off_words[SEC_ROW_IV]);
  const int ns = a.n_seg ? a.n_seg[b] : 0;
  int seg = -1;
  if (ns > 0 && ns <= a.seg_cap) {
    const int32_t* bd = a.seg_bounds + size_t(b) * (a.seg_cap + 1);
    int lo = 0, hi = ns - 1;  // the last segment starting at or before x
    if (bd[0] <= x) {
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bd[mid] <= x) lo = mid; else hi = mid - 1;
      }
      if (x < bd[lo + 1]) seg = lo;
    }
  }
  out[t] = seg;
}

__global__ __launch_bounds__(kThreads) void blockmask_kernel(PreprocessArgs a, int family) {
  extern __shared__ int32_t lds[];
  const int b = blockIdx.y;
  const bool row_role = int(blockIdx.x) < a.Tq_f;
  const int tile = row_role ? int(blockIdx.x) : int(blockIdx.x) - a.Tq_f;
  uint32_t* desc = a.desc;
  const int N = a.N;
  const int x0 = tile * (row_role ? a.fq : a.bk);
  const int nx = min(row_role ? a.fq : a.bk, N - x0);   // this tile's rows (or keys)
  const int Bt = row_role ? a.fk : a.bq;                 // tile width along the other axis
  const int T = row_role ? a.Tk_f : a.Tq_b;
  const int W = row_role ? a.Wf : a.Wb;
  int32_t* cnt = lds;                  // [T]
  int32_t* own_seg = lds + T;          // [nx] segments of this tile's indices
  int32_t* misc = own_seg + 128;       // [0] sample error, [1] error OR over samples

  const int tid = threadIdx.x;
  for (int t = tid; t < T; t += kThreads) cnt[t] = 0;
  const int32_t* tok = reinterpret_cast<const int32_t*>(desc + a.off_words[SEC_ROW_IV]) + size_t(b) * N;
  for (int t = tid; t < nx; t += kThreads) own_seg[t] = tok[x0 + t];
  if (tid == 0) {
    const int ns = a.n_seg ? a.n_seg[b] : 0;
    misc[0] = int32_t(validate_sample(N, ns, a.seg_cap, a.seg_bounds ? a.seg_bounds + size_t(b) * (a.seg_cap + 1) : nullptr,
                                      a.refs ? a.refs + size_t(b) * a.seg_cap * a.n_refs : nullptr, a.n_refs));
    misc[1] = 0;
  }
  __syncthreads();
  if (blockIdx.x == 0 && b == 0) {
    for (int bb = tid; bb < a.B; bb += kThreads) {
      const int ns = a.n_seg ? a.n_seg[bb] : 0;
      const uint32_t e = validate_sample(N, ns, a.seg_cap,
                                         a.seg_bounds ? a.seg_bounds + size_t(bb) * (a.seg_cap + 1) : nullptr,
                                         a.refs ? a.refs + size_t(bb) * a.seg_cap * a.n_refs : nullptr, a.n_refs);
      atomicOr(reinterpret_cast<uint32_t*>(&misc[1]), e);
    }
  }

  const uint32_t err = uint32_t(misc[0]);
  PredSample ps;
  ps.family = family;
  ps.N = N;
  ps.n_refs = a.n_refs;
  ps.valid = err == 0u;
  ps.scalar = a.n_scalars > 0 ? a.scalars[size_t(b) * a.n_scalars] : 0;
  ps.seg = tok;
  ps.refs = a.refs ? a.refs + size_t(b) * a.seg_cap * a.n_refs : nullptr;

  // every element of this tile row: one index of the other axis per thread
  for (int y = tid; y < N; y += kThreads) {
    int count = 0;
    const int sy = tok[y];
    if (row_role) {
      for (int r = 0; r < nx; ++r) count += pred_visible(ps, x0 + r, y, own_seg[r], sy) ? 1 : 0;
    } else {
      for (int r = 0; r < nx; ++r) count += pred_visible(ps, y, x0 + r, sy, own_seg[r]) ? 1 : 0;
    }
    if (count) atomicAdd(&cnt[y / Bt], count);
  }
  __syncthreads();
  uint32_t* bitmap = desc + a.off_words[row_role ? SEC_FBM : SEC_BBM] + (size_t(b) * (row_role ? a.Tq_f : a.Tk_b) + tile) * W;
  for (int w = tid; w < W; w += kThreads) {
    uint32_t word = 0;
    for (int t = 16 * w; t < min(T, 16 * w + 16); ++t) {
      const int area = nx * min(Bt, N - t * Bt);
      const uint32_t code = cnt[t] == 0 ? 0u : (cnt[t] == area ? 1u : 2u);
      word |= code << (2 * (t - 16 * w));
    }
    bitmap[w] = word;
  }
  if (tid == 0) {
    (row_role ? desc[a.off_words[SEC_ROW_TKMAX] + size_t(b) * a.Tq_f + tile]
              : desc[a.off_words[SEC_COL_TKMAX] + size_t(b) * a.Tk_b + tile]) = 0u;
    if (blockIdx.x == 0) desc[a.off_words[SEC_SAMPLE_ERR] + b] = err;
    if (blockIdx.x == 0 && b == 0) {
      uint4* h = reinterpret_cast<uint4*>(desc + a.off_words[SEC_HEADER]);
      h[0] = make_uint4(CM_DESC_MAGIC, uint32_t(a.B), uint32_t(a.N), uint32_t(a.K_r));
      h[1] = make_uint4(uint32_t(a.K_c), uint32_t(a.fq), uint32_t(a.fk), uint32_t(a.bk));
      h[2] = make_uint4(uint32_t(a.bq), uint32_t(a.Tq_f), uint32_t(a.Tk_f), uint32_t(a.Tk_b));
      h[3] = make_uint4(uint32_t(a.Tq_b), uint32_t(misc[1]), uint32_t(a.seg_cap), 0u);
    }
  }
}

}  // namespace

hipError_t launch_blockmask(const PreprocessArgs& a, int family, hipStream_t stream) {
  const int64_t tokens = int64_t(a.B) * a.N;
  hipLaunchKernelGGL(tok_seg_kernel, dim3(unsigned((tokens + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int T = a.Tk_f > a.Tq_b ? a.Tk_f : a.Tq_b;
  const size_t lds = sizeof(int32_t) * (size_t(T) + 128 + 2);
  hipLaunchKernelGGL(blockmask_kernel, dim3(a.Tq_f + a.Tk_b, a.B), dim3(kThreads), lds, stream, a, family);
  return hipGetLastError();
}

}  // namespace cm
