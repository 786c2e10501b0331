// api.cpp -- the C ABI: argument checks, descriptor layout, kernel launches.
//
// Every entry point validates its arguments on the host before it enqueues
// anything; a failed check returns a negative cm_status and launches nothing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"

namespace cm {

cm_status compile_spec(const char* text, cm_spec** out);

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

cm_status fail(cm_status st, const std::string& msg) {
  g_error = msg;
  return st;
}

namespace {

constexpr int kMaxTiles = 4096;          // tiles along one axis (LDS of the preprocess)
constexpr size_t kMaxPreprocessLds = 64 * 1024;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int cdiv(int a, int b) { return (a + b - 1) / b; }

cm_status fill_layout(cm_desc& d) {
  const cm_tiles& t = d.tiles;
  d.Tq_f = cdiv(d.N, t.fwd_q);
  d.Tk_f = cdiv(d.N, t.fwd_k);
  d.Tk_b = cdiv(d.N, t.bwd_k);
  d.Tq_b = cdiv(d.N, t.bwd_q);
  d.Wf = cdiv(d.Tk_f, 16);
  d.Wb = cdiv(d.Tq_b, 16);
  if (d.Tk_f > kMaxTiles || d.Tq_b > kMaxTiles)
    return fail(CM_ERR_INVALID, "more than 4096 tiles along one axis; use larger tiles");
  const size_t B = size_t(d.B), N = size_t(d.N);
  const size_t sizes[8] = {16 * 4,
                           size_t(d.packed ? d.packed : d.B) * 4,
                           B * d.Tq_f * 4,
                           B * d.Tk_b * 4,
                           B * d.Tq_f * d.Wf * 4,
                           B * d.Tk_b * d.Wb * 4,
                           B * N * d.K_r * 8,
                           B * N * d.K_c * 8};
  size_t pos = 0;
  for (int s = 0; s < 8; ++s) {
    d.off[s] = pos;
    pos = align256(pos + sizes[s]);
  }
  d.off[SEC_TOTAL] = pos;
  return CM_OK;
}

cm_status make_layout(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap, const cm_tiles* tiles, cm_desc& d,
                      int32_t packed = 0) {
  if (!spec || !tiles) return fail(CM_ERR_NULL, "spec and tiles are required");
  if (B < 1 || N < 1) return fail(CM_ERR_INVALID, "B and N must be >= 1");
  if (packed < 0 || packed > (1 << 20)) return fail(CM_ERR_INVALID, "n_samples must be in [1, 2^20]");
  d.packed = packed;
  if (N > (1 << 28)) return fail(CM_ERR_INVALID, "N must be below 2^28");
  if (seg_cap < 0 || seg_cap > 4096) return fail(CM_ERR_INVALID, "seg_cap must be in [0, 4096]");
  if (tiles->fwd_q < 1 || tiles->fwd_k < 1 || tiles->bwd_k < 1 || tiles->bwd_q < 1)
    return fail(CM_ERR_INVALID, "tile sizes must be >= 1");
  d.spec_id = spec->id;
  d.B = B;
  d.N = N;
  d.seg_cap = seg_cap;
  d.tiles = *tiles;
  d.K_r = spec_width(spec, 0, seg_cap);
  d.K_c = spec_width(spec, 1, seg_cap);
  cm_status st = fill_layout(d);
  if (st != CM_OK) return st;
  const int Tmax = std::max(d.Tk_f, d.Tq_b);
  const size_t lds = 4 * (size_t(2) * (Tmax + 1) + 2 * 256 + 4 + (seg_cap + 1) + size_t(seg_cap) * spec->n_refs +
                          spec->params.size());
  if (lds > kMaxPreprocessLds) return fail(CM_ERR_INVALID, "metadata capacity and tile counts exceed the preprocess LDS budget");
  return CM_OK;
}

cm_status hip_fail(hipError_t e, const char* where) {
  return fail(CM_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

DescView desc_view(const cm_desc* d) {
  DescView v;
  const uint8_t* base = static_cast<const uint8_t*>(d->buf);
  v.fbm = reinterpret_cast<const uint32_t*>(base + d->off[SEC_FBM]);
  v.bbm = reinterpret_cast<const uint32_t*>(base + d->off[SEC_BBM]);
  v.row_iv = reinterpret_cast<const uint32_t*>(base + d->off[SEC_ROW_IV]);
  v.col_iv = reinterpret_cast<const uint32_t*>(base + d->off[SEC_COL_IV]);
  v.row_tkmax = reinterpret_cast<const uint32_t*>(base + d->off[SEC_ROW_TKMAX]);
  v.col_tkmax = reinterpret_cast<const uint32_t*>(base + d->off[SEC_COL_TKMAX]);
  v.K_r = d->K_r; v.K_c = d->K_c; v.Wf = d->Wf; v.Wb = d->Wb;
  v.Tq_f = d->Tq_f; v.Tk_f = d->Tk_f; v.Tk_b = d->Tk_b; v.Tq_b = d->Tq_b;
  v.fq = d->tiles.fwd_q; v.fk = d->tiles.fwd_k; v.bk = d->tiles.bwd_k; v.bq = d->tiles.bwd_q;
  v.packed = d->packed;
  std::memset(&v.pred, 0, sizeof(v.pred));
  v.pred.family = d->family;
  if (d->family >= 0) {
    v.pred.tok_seg = reinterpret_cast<const int32_t*>(base + d->off[SEC_ROW_IV]);
    v.pred.scalars = d->pred_md.scalars;
    v.pred.n_scalars = d->pred_md.n_scalars;
    v.pred.refs = d->seg_cap > 0 ? d->pred_md.refs : nullptr;
    v.pred.seg_cap = d->seg_cap;
    v.pred.n_refs = d->seg_cap > 0 ? d->pred_md.n_refs : 0;
    v.pred.sample_err = reinterpret_cast<const uint32_t*>(base + d->off[SEC_SAMPLE_ERR]);
  }
  return v;
}

// Checks shared by the attention entry points.  Fills dims and the descriptor
// view; in causal mode the view carries the default tile shape only.
cm_status check_attn(const cm_attn_args* args, const cm_desc* desc, AttnDims& dims, DescView& view) {
  if (!args) return fail(CM_ERR_NULL, "args is NULL");
  if (args->B < 1 || args->H < 1 || args->N < 1) return fail(CM_ERR_INVALID, "B, H, N must be >= 1");
  if (args->d != 64 && args->d != 128) return fail(CM_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  dims.B = args->B; dims.H = args->H; dims.N = args->N; dims.d = args->d;
  if (args->stride_b == 0 && args->stride_h == 0 && args->stride_n == 0) {
    dims.sn = args->d;
    dims.sh = int64_t(args->N) * args->d;
    dims.sb = int64_t(args->H) * dims.sh;
  } else {
    dims.sb = args->stride_b; dims.sh = args->stride_h; dims.sn = args->stride_n;
    if (dims.sn < args->d || dims.sh < 1 || dims.sb < 1 || dims.sn % 8 || dims.sh % 8 || dims.sb % 8)
      return fail(CM_ERR_INVALID, "strides must be positive multiples of 8 elements with stride_n >= d");
  }
  // the largest grid (rowsum(dO * O), 16 lanes per row) has 16 * B * H * N
  // work-items, which must stay below 2^32; each head's rows are addressed
  // through one buffer descriptor, whose size field has 32 bits
  if (int64_t(args->B) * args->H * args->N > (int64_t(1) << 27))
    return fail(CM_ERR_UNSUPPORTED, "B * H * N must be at most 2^27 rows per call");
  if (((int64_t(args->N) - 1) * dims.sn + args->d) * 2 > int64_t(UINT32_MAX))
    return fail(CM_ERR_UNSUPPORTED, "one head's rows ((N - 1) * stride_n + d bf16) must span less than 4 GiB");
  if (!std::isfinite(args->scale) || args->scale < 0) return fail(CM_ERR_INVALID, "scale must be finite and >= 0");
  dims.scale = args->scale == 0.f ? 1.0f / std::sqrt(float(args->d)) : args->scale;
  dims.causal = args->causal ? 1 : 0;
  if (args->check != CM_CHECK_RUN_BITS && args->check != CM_CHECK_ORDINARY_MASKED && args->check != CM_CHECK_PREDICATE &&
      args->check != CM_CHECK_UNSIGNED)
    return fail(CM_ERR_INVALID, "check must be CM_CHECK_RUN_BITS (0), CM_CHECK_ORDINARY_MASKED (1), CM_CHECK_PREDICATE (2) "
                                "or CM_CHECK_UNSIGNED (3)");
  dims.check = args->check;
  if (args->precision != CM_PRECISION_BF16 && args->precision != CM_PRECISION_SPLIT)
    return fail(CM_ERR_INVALID, "precision must be CM_PRECISION_BF16 (0) or CM_PRECISION_SPLIT (1)");
  if (args->precision == CM_PRECISION_SPLIT && args->check != CM_CHECK_RUN_BITS)
    return fail(CM_ERR_UNSUPPORTED, "CM_PRECISION_SPLIT runs with the default check (CM_CHECK_RUN_BITS) only");
  dims.precision = args->precision;
  if (args->check == CM_CHECK_PREDICATE && dims.causal)
    return fail(CM_ERR_INVALID, "the predicate baseline runs on a block-mask descriptor, not the maskless causal path");
  std::memset(&view, 0, sizeof(view));
  if (dims.causal) {
    view.fq = 128; view.fk = 64; view.bk = 128; view.bq = 64;
    if (args->d == 64 && args->N <= 256) { view.fq = 64; view.bk = 64; }
    view.Tq_f = cdiv(args->N, view.fq); view.Tk_f = cdiv(args->N, view.fk);
    view.Tk_b = cdiv(args->N, view.bk); view.Tq_b = cdiv(args->N, view.bq);
    return CM_OK;
  }
  if (!desc) return fail(CM_ERR_NULL, "desc is NULL (only the causal path runs without a descriptor)");
  if (desc->B != args->B || desc->N != args->N)
    return fail(CM_ERR_MISMATCH, "descriptor was built for B=" + std::to_string(desc->B) + ", N=" + std::to_string(desc->N));
  if (!attn_tiles_supported(args->d, desc->tiles.fwd_q, desc->tiles.fwd_k, desc->tiles.bwd_k, desc->tiles.bwd_q))
    return fail(CM_ERR_UNSUPPORTED, "descriptor tile shape has no attention kernel (supported: forward 64x64 or "
                                    "128x64, backward 64x64 or 128x64)");
  if ((args->check == CM_CHECK_PREDICATE) != (desc->family >= 0))
    return fail(CM_ERR_MISMATCH, desc->family >= 0 ? "a block-mask descriptor (cm_build_blockmask) needs check = CM_CHECK_PREDICATE"
                                                  : "check = CM_CHECK_PREDICATE needs a block-mask descriptor (cm_build_blockmask)");
  view = desc_view(desc);
  return CM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace cm

using namespace cm;

extern "C" {

cm_status cm_spec_compile(const char* text, cm_spec** out) {
  if (!text || !out) return fail(CM_ERR_NULL, "text and out are required");
  *out = nullptr;
  return compile_spec(text, out);
}

void cm_spec_free(cm_spec* spec) { delete spec; }

cm_status cm_spec_info(const cm_spec* spec, int32_t seg_cap, int32_t* K_row, int32_t* K_col, int32_t* n_scalars,
                       int32_t* n_refs) {
  if (!spec) return fail(CM_ERR_NULL, "spec is NULL");
  if (seg_cap < 0) return fail(CM_ERR_INVALID, "seg_cap must be >= 0");
  if (K_row) *K_row = spec_width(spec, 0, seg_cap);
  if (K_col) *K_col = spec_width(spec, 1, seg_cap);
  if (n_scalars) *n_scalars = int32_t(spec->params.size());
  if (n_refs) *n_refs = spec->n_refs;
  return CM_OK;
}

cm_status cm_spec_dump(const cm_spec* spec, char* buf, size_t len, size_t* needed) {
  if (!spec) return fail(CM_ERR_NULL, "spec is NULL");
  if (needed) *needed = spec->listing.size() + 1;
  if (buf && len) {
    size_t n = std::min(len - 1, spec->listing.size());
    std::memcpy(buf, spec->listing.data(), n);
    buf[n] = 0;
  }
  return CM_OK;
}

cm_status cm_spec_eval_host(const cm_spec* spec, int32_t direction, int32_t N, int32_t index, const int32_t* scalars,
                            int32_t n_scalars, const int32_t* seg_bounds, int32_t n_seg, int32_t seg_cap,
                            const int32_t* refs, int32_t n_refs, uint32_t* runs, int32_t cap, int32_t* n_runs,
                            uint32_t* md_err) {
  if (!spec || !runs || !n_runs || !md_err) return fail(CM_ERR_NULL, "spec, runs, n_runs, md_err are required");
  if (direction != 0 && direction != 1) return fail(CM_ERR_INVALID, "direction must be 0 or 1");
  if (N < 1 || index < 0 || index >= N) return fail(CM_ERR_INVALID, "index out of range");
  if (n_scalars < int32_t(spec->params.size())) return fail(CM_ERR_MISMATCH, "too few scalars for the spec");
  if (n_refs < spec->n_refs) return fail(CM_ERR_MISMATCH, "too few references per segment for the spec");
  if (seg_cap < 0) return fail(CM_ERR_INVALID, "seg_cap must be >= 0");
  if ((seg_cap > 0 && !seg_bounds) || (n_refs > 0 && seg_cap > 0 && !refs) || (n_scalars > 0 && !scalars))
    return fail(CM_ERR_NULL, "metadata array missing");
  *md_err = (n_seg < 0 || n_seg > seg_cap) ? 1u : validate_sample(N, n_seg, seg_cap, seg_bounds, refs, n_refs);
  *n_runs = 0;
  if (*md_err) return CM_OK;
  SampleView sv;
  sv.N = N; sv.n_seg = n_seg; sv.n_refs = n_refs; sv.scalars = scalars; sv.bounds = seg_bounds; sv.refs = refs;
  std::vector<std::pair<uint32_t, uint32_t>> iv;
  eval_direction(spec->prog.w, spec->dir_off[direction], sv, index,
                 [&](int32_t lo, int32_t hi) { iv.emplace_back(uint32_t(lo), uint32_t(hi)); });
  std::stable_sort(iv.begin(), iv.end(), [](const std::pair<uint32_t, uint32_t>& x, const std::pair<uint32_t, uint32_t>& y) {
    return x.first < y.first;
  });
  std::vector<std::pair<uint32_t, uint32_t>> merged;
  for (auto& p : iv) {
    if (!merged.empty() && p.first <= merged.back().second) merged.back().second = std::max(merged.back().second, p.second);
    else merged.push_back(p);
  }
  if (int32_t(merged.size()) > cap) return fail(CM_ERR_SIZE, "runs buffer too small");
  for (size_t q = 0; q < merged.size(); ++q) { runs[2 * q] = merged[q].first; runs[2 * q + 1] = merged[q].second; }
  *n_runs = int32_t(merged.size());
  return CM_OK;
}

cm_status cm_desc_size(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap, const cm_tiles* tiles, size_t* bytes) {
  if (!bytes) return fail(CM_ERR_NULL, "bytes is NULL");
  cm_desc d;
  cm_status st = make_layout(spec, B, N, seg_cap, tiles, d);
  if (st != CM_OK) return st;
  *bytes = d.off[SEC_TOTAL];
  return CM_OK;
}

static cm_status desc_init(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap, const cm_tiles* tiles,
                           void* dev_buf, size_t bytes, cm_desc** out, int32_t packed) {
  if (!out || !dev_buf) return fail(CM_ERR_NULL, "dev_buf and out are required");
  *out = nullptr;
  cm_desc d;
  cm_status st = make_layout(spec, B, N, seg_cap, tiles, d, packed);
  if (st != CM_OK) return st;
  if (bytes < d.off[SEC_TOTAL])
    return fail(CM_ERR_SIZE, "descriptor buffer has " + std::to_string(bytes) + " bytes, needs " +
                                 std::to_string(d.off[SEC_TOTAL]));
  if (reinterpret_cast<uintptr_t>(dev_buf) & 255) return fail(CM_ERR_INVALID, "descriptor buffer must be 256-byte aligned");
  hipError_t e = hipMemsetAsync(dev_buf, 0, d.off[SEC_TOTAL], nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return hip_fail(e, "cm_desc_init");
  d.buf = dev_buf;
  d.bytes = bytes;
  *out = new cm_desc(d);
  return CM_OK;
}

cm_status cm_desc_init(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap, const cm_tiles* tiles, void* dev_buf,
                       size_t bytes, cm_desc** out) {
  return desc_init(spec, B, N, seg_cap, tiles, dev_buf, bytes, out, 0);
}

cm_status cm_desc_size_packed(const cm_spec* spec, int32_t n_samples, int32_t T, int32_t seg_cap, const cm_tiles* tiles,
                              size_t* bytes) {
  if (!bytes) return fail(CM_ERR_NULL, "bytes is NULL");
  if (n_samples < 1) return fail(CM_ERR_INVALID, "n_samples must be >= 1");
  cm_desc d;
  cm_status st = make_layout(spec, 1, T, seg_cap, tiles, d, n_samples);
  if (st != CM_OK) return st;
  *bytes = d.off[SEC_TOTAL];
  return CM_OK;
}

cm_status cm_desc_init_packed(const cm_spec* spec, int32_t n_samples, int32_t T, int32_t seg_cap, const cm_tiles* tiles,
                              void* dev_buf, size_t bytes, cm_desc** out) {
  if (n_samples < 1) return fail(CM_ERR_INVALID, "n_samples must be >= 1");
  return desc_init(spec, 1, T, seg_cap, tiles, dev_buf, bytes, out, n_samples);
}

void cm_desc_free(cm_desc* desc) { delete desc; }

cm_status cm_desc_offsets(const cm_desc* desc, size_t* offsets) {
  if (!desc || !offsets) return fail(CM_ERR_NULL, "desc and offsets are required");
  for (int s = 0; s < 9; ++s) offsets[s] = desc->off[s];
  return CM_OK;
}

cm_status cm_build_blockmask(int32_t family, const cm_metadata* md, cm_desc* desc, cm_stream stream) {
  if (!md || !desc) return fail(CM_ERR_NULL, "md and desc are required");
  if (family < CM_PRED_CAUSAL || family > CM_PRED_RETRIEVAL) return fail(CM_ERR_INVALID, "unknown predicate family");
  if (desc->packed) return fail(CM_ERR_UNSUPPORTED, "the predicate baseline covers padded batches only");
  if (md->cu_seqlens) return fail(CM_ERR_MISMATCH, "the predicate baseline covers padded batches only");
  const int need_scalars = family == CM_PRED_CAUSAL ? 0 : 1;
  const int need_refs = family == CM_PRED_RETRIEVAL ? 1 : 0;
  if (md->n_scalars < need_scalars || (need_scalars && !md->scalars))
    return fail(CM_ERR_MISMATCH, "this family reads one per-sample scalar (metadata scalars[b][0])");
  if (md->n_refs < 0 || md->n_refs > 2) return fail(CM_ERR_UNSUPPORTED, "the predicate baseline reads at most 2 references per segment");
  if (need_refs && desc->seg_cap > 0 && md->n_refs > 0 && !md->refs) return fail(CM_ERR_NULL, "refs is NULL");
  if (desc->seg_cap > 0 && (!md->seg_bounds || !md->n_seg)) return fail(CM_ERR_NULL, "seg_bounds and n_seg are required");
  if (desc->K_r < 1) return fail(CM_ERR_UNSUPPORTED, "the descriptor's row table is empty (K_row 0): no room for token segments");
  if (desc->tiles.fwd_q > 128 || desc->tiles.bwd_k > 128)
    return fail(CM_ERR_UNSUPPORTED, "block masks are built for tiles of at most 128 query rows / keys");
  PreprocessArgs a;
  std::memset(&a, 0, sizeof(a));
  a.scalars = md->scalars;
  a.seg_bounds = desc->seg_cap > 0 ? md->seg_bounds : nullptr;
  a.n_seg = desc->seg_cap > 0 ? md->n_seg : nullptr;
  a.refs = (desc->seg_cap > 0 && md->n_refs > 0) ? md->refs : nullptr;
  a.n_scalars = md->n_scalars;
  a.n_refs = (desc->seg_cap > 0) ? md->n_refs : 0;
  a.seg_cap = desc->seg_cap;
  a.desc = static_cast<uint32_t*>(desc->buf);
  a.B = desc->B; a.N = desc->N; a.K_r = desc->K_r; a.K_c = desc->K_c;
  a.fq = desc->tiles.fwd_q; a.fk = desc->tiles.fwd_k; a.bk = desc->tiles.bwd_k; a.bq = desc->tiles.bwd_q;
  a.Tq_f = desc->Tq_f; a.Tk_f = desc->Tk_f; a.Tk_b = desc->Tk_b; a.Tq_b = desc->Tq_b; a.Wf = desc->Wf; a.Wb = desc->Wb;
  for (int s = 0; s < 8; ++s) a.off_words[s] = uint32_t(desc->off[s] / 4);
  hipError_t e = launch_blockmask(a, family, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cm_build_blockmask");
  desc->family = family;
  desc->pred_md = *md;
  return CM_OK;
}

cm_status cm_build_descriptor(const cm_spec* spec, const cm_metadata* md, cm_desc* desc, cm_stream stream) {
  if (!spec || !md || !desc) return fail(CM_ERR_NULL, "spec, md and desc are required");
  if (desc->spec_id != spec->id) return fail(CM_ERR_MISMATCH, "descriptor was initialised for another spec");
  if (md->n_scalars < int32_t(spec->params.size()))
    return fail(CM_ERR_MISMATCH, "metadata has " + std::to_string(md->n_scalars) + " scalars, the spec needs " +
                                     std::to_string(spec->params.size()));
  if (md->n_refs < spec->n_refs) return fail(CM_ERR_MISMATCH, "metadata carries fewer references than the spec uses");
  if (md->n_refs > kMaxRefs) return fail(CM_ERR_INVALID, "at most 15 references per segment");
  if (md->n_scalars > 0 && !md->scalars) return fail(CM_ERR_NULL, "scalars is NULL");
  if (desc->seg_cap > 0 && (!md->seg_bounds || !md->n_seg)) return fail(CM_ERR_NULL, "seg_bounds and n_seg are required");
  if (desc->seg_cap > 0 && md->n_refs > 0 && !md->refs) return fail(CM_ERR_NULL, "refs is NULL");
  if (desc->packed && !md->cu_seqlens) return fail(CM_ERR_NULL, "a packed descriptor needs md->cu_seqlens");
  if (!desc->packed && md->cu_seqlens)
    return fail(CM_ERR_MISMATCH, "md->cu_seqlens is set but the descriptor is not packed (cm_desc_init_packed)");
  const size_t lds = 4 * (size_t(2) * (std::max(desc->Tk_f, desc->Tq_b) + 1) + 2 * 256 + 4 + (desc->seg_cap + 1) +
                          size_t(desc->seg_cap) * md->n_refs + md->n_scalars);
  if (lds > kMaxPreprocessLds) return fail(CM_ERR_INVALID, "metadata too large for the preprocess LDS budget");
  PreprocessArgs a;
  std::memset(&a, 0, sizeof(a));
  a.scalars = md->scalars;
  a.seg_bounds = desc->seg_cap > 0 ? md->seg_bounds : nullptr;
  a.n_seg = md->n_seg;
  a.refs = (desc->seg_cap > 0 && md->n_refs > 0) ? md->refs : nullptr;
  a.cu_seqlens = desc->packed ? md->cu_seqlens : nullptr;
  a.n_samples = desc->packed;
  a.n_scalars = md->n_scalars;
  a.n_refs = (desc->seg_cap > 0) ? md->n_refs : 0;
  a.seg_cap = desc->seg_cap;
  a.desc = static_cast<uint32_t*>(desc->buf);
  a.B = desc->B; a.N = desc->N; a.K_r = desc->K_r; a.K_c = desc->K_c;
  a.fq = desc->tiles.fwd_q; a.fk = desc->tiles.fwd_k; a.bk = desc->tiles.bwd_k; a.bq = desc->tiles.bwd_q;
  a.Tq_f = desc->Tq_f; a.Tk_f = desc->Tk_f; a.Tk_b = desc->Tk_b; a.Tq_b = desc->Tq_b; a.Wf = desc->Wf; a.Wb = desc->Wb;
  for (int s = 0; s < 8; ++s) a.off_words[s] = uint32_t(desc->off[s] / 4);
  a.dir_off[0] = spec->dir_off[0];
  a.dir_off[1] = spec->dir_off[1];
  void* fn = specialized_function(spec);
  hipError_t e = fn ? launch_specialized(fn, a, static_cast<hipStream_t>(stream))
                    : launch_preprocess(a, spec->prog, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cm_build_descriptor");
  desc->family = -1;
  return CM_OK;
}

cm_status cm_attn_fwd(const cm_attn_args* args, const void* q, const void* k, const void* v, const cm_desc* desc, void* o,
                      float* lse, cm_stream stream) {
  AttnDims dims;
  DescView view;
  cm_status st = check_attn(args, desc, dims, view);
  if (st != CM_OK) return st;
  if (!q || !k || !v || !o || !lse) return fail(CM_ERR_NULL, "q, k, v, o, lse are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return fail(CM_ERR_INVALID, "tensors must be 16-byte aligned");
  hipError_t e = launch_attn_fwd(dims, q, k, v, view, o, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cm_attn_fwd");
  return CM_OK;
}

cm_status cm_attn_bwd_workspace(const cm_attn_args* args, size_t* bytes) {
  if (!args || !bytes) return fail(CM_ERR_NULL, "args and bytes are required");
  if (args->B < 1 || args->H < 1 || args->N < 1) return fail(CM_ERR_INVALID, "B, H, N must be >= 1");
  *bytes = 2 * size_t(args->B) * args->H * args->N * sizeof(float);
  return CM_OK;
}

// dK/dV and dQ both depend only on D.  Where the backward grid is short,
// the dK/dV launch ends in a tail of long work-groups (the first key tiles of
// lower-triangular masks), and dQ launched on a second stream fills the CUs
// that tail leaves idle.  One side stream and two events per device, created
// on first use; the mutex keeps each call's record/wait pairs together.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
static std::mutex g_side_mu;
static SideStream g_side[kMaxSideDevices];

// *out stays null (and the caller runs the backward on its own stream) when
// the side stream does not exist yet and the caller's stream is being
// captured: nothing is created inside a capture.
static hipError_t side_stream(hipStream_t caller, SideStream** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(caller, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipSuccess;
    SideStream made;
    e = hipStreamCreateWithFlags(&made.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&made.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&made.join, hipEventDisableTiming);
    if (e != hipSuccess) {  // keep nothing half made; a later call tries again
      if (made.fork) (void)hipEventDestroy(made.fork);
      if (made.stream) (void)hipStreamDestroy(made.stream);
      return e;
    }
    ss = made;
  }
  *out = &ss;
  return hipSuccess;
}

// Run dQ beside dK/dV when the dK/dV grid has at most two 256-key
// work-groups per CU (each holds a whole CU).  Measured on MI355X: 7-8% off
// the backward of B4 H8 N4096 HSTU batches (2 per CU); within noise for
// causal (4 per CU), packed HSTU and retrieval batches (8 per CU); 5% slower
// for B1 H16 N32768 reward-model batches (8 per CU), whose long key columns
// then share each XCD's L2 and power budget with dQ.
constexpr int64_t kComputeUnits = 256;
static bool overlap_backward(const AttnDims& a) {
  return int64_t(a.B) * a.H * a.N <= 2 * kComputeUnits * 256;
}

static cm_status bwd_run(int32_t stage, const cm_attn_args* args, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dO, const cm_desc* desc, void* dq, void* dk,
                         void* dv, void* workspace, size_t workspace_bytes, bool fixed_scratch, cm_stream stream) {
  AttnDims dims;
  DescView view;
  cm_status st = check_attn(args, desc, dims, view);
  if (st != CM_OK) return st;
  if (stage < -1 || stage > 2) return fail(CM_ERR_INVALID, "stage must be 0, 1 or 2");
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || (!fixed_scratch && !workspace))
    return fail(CM_ERR_NULL, fixed_scratch ? "q, k, v, o, lse, dO, dq, dk and dv are required"
                                           : "q, k, v, o, lse, dO, dq, dk, dv and workspace are required");
  size_t need = 0;
  cm_attn_bwd_workspace(args, &need);
  if (fixed_scratch) {
    const size_t rows = size_t(args->B) * args->H * args->N;
    if (rows > kScratchRows)
      return fail(CM_ERR_SIZE, "cm_attn_bwd_noalloc covers at most " + std::to_string(kScratchRows) +
                                   " rows (B * H * N); this call has " + std::to_string(rows));
  } else if (workspace_bytes < need) {
    return fail(CM_ERR_SIZE, "workspace needs " + std::to_string(need) + " bytes");
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (!fixed_scratch && !aligned16(workspace)))
    return fail(CM_ERR_INVALID, "tensors must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* D = static_cast<float*>(workspace);
  hipError_t e = hipSuccess;
  if (fixed_scratch) {
    e = scratch_workspace(&D);
    if (e != hipSuccess) return hip_fail(e, "cm_attn_bwd_noalloc (scratch address)");
  }
  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (stage == -1 && !fixed_scratch && overlap_backward(dims)) {
    lock.lock();
    e = side_stream(s, &ss);
    if (e != hipSuccess) return hip_fail(e, "cm_attn_bwd (side stream)");
  }
  if (ss) {
    e = launch_bwd_dot(dims, o, dO, lse, D, s);
    if (e == hipSuccess) e = hipEventRecord(ss->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
    if (e == hipSuccess) e = launch_bwd_dkdv(dims, q, k, v, lse, dO, D, view, dk, dv, s);
    if (e == hipSuccess) e = launch_bwd_dq(dims, q, k, v, lse, dO, D, view, dq, ss->stream);
    if (e == hipSuccess) e = hipEventRecord(ss->join, ss->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->join, 0);
  } else {
    if (stage == -1 || stage == 0) e = launch_bwd_dot(dims, o, dO, lse, D, s);
    if (e == hipSuccess && (stage == -1 || stage == 1)) e = launch_bwd_dkdv(dims, q, k, v, lse, dO, D, view, dk, dv, s);
    if (e == hipSuccess && (stage == -1 || stage == 2)) e = launch_bwd_dq(dims, q, k, v, lse, dO, D, view, dq, s);
  }
  if (e != hipSuccess) return hip_fail(e, fixed_scratch ? "cm_attn_bwd_noalloc" : "cm_attn_bwd");
  return CM_OK;
}

cm_status cm_attn_bwd_stage(int32_t stage, const cm_attn_args* args, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dO, const cm_desc* desc, void* dq, void* dk,
                            void* dv, void* workspace, size_t workspace_bytes, cm_stream stream) {
  return bwd_run(stage, args, q, k, v, o, lse, dO, desc, dq, dk, dv, workspace, workspace_bytes, false, stream);
}

cm_status cm_attn_bwd(const cm_attn_args* args, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, const cm_desc* desc, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, cm_stream stream) {
  return bwd_run(-1, args, q, k, v, o, lse, dO, desc, dq, dk, dv, workspace, workspace_bytes, false, stream);
}

cm_status cm_attn_bwd_noalloc(const cm_attn_args* args, const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, const cm_desc* desc, void* dq, void* dk, void* dv,
                              cm_stream stream) {
  return bwd_run(-1, args, q, k, v, o, lse, dO, desc, dq, dk, dv, nullptr, 0, true, stream);
}

cm_status cm_desc_download(const cm_desc* desc, void* host, size_t bytes, cm_stream stream) {
  if (!desc || !host) return fail(CM_ERR_NULL, "desc and host are required");
  const size_t total = desc->off[SEC_TOTAL];
  if (bytes < total) return fail(CM_ERR_SIZE, "host buffer has " + std::to_string(bytes) + " bytes, the descriptor " +
                                                  std::to_string(total));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(host, desc->buf, total, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "cm_desc_download");
  return CM_OK;
}

cm_status cm_desc_errors(const cm_desc* desc, uint32_t* flags, uint32_t* per_sample, int32_t* n_per_sample,
                         cm_stream stream) {
  if (!desc || !flags) return fail(CM_ERR_NULL, "desc and flags are required");
  const int32_t n = desc->packed ? desc->packed : desc->B;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* base = static_cast<const uint8_t*>(desc->buf);
  uint32_t header[16];
  hipError_t e = hipMemcpyAsync(header, base, sizeof(header), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && per_sample)
    e = hipMemcpyAsync(per_sample, base + desc->off[SEC_SAMPLE_ERR], size_t(n) * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "cm_desc_errors");
  *flags = header[13];
  if (n_per_sample) *n_per_sample = n;
  return CM_OK;
}

const char* cm_status_str(cm_status status) {
  switch (status) {
    case CM_OK: return "ok";
    case CM_ERR_NULL: return "null pointer";
    case CM_ERR_INVALID: return "invalid argument";
    case CM_ERR_PARSE: return "spec parse/lowering error";
    case CM_ERR_MISMATCH: return "descriptor/spec/argument mismatch";
    case CM_ERR_UNSUPPORTED: return "unsupported shape";
    case CM_ERR_SIZE: return "buffer too small";
    case CM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* cm_last_error(void) { return g_error.c_str(); }

const char* cm_version(void) { return "compilemask-mi355x 0.1 (gfx950)"; }

}  // extern "C"
