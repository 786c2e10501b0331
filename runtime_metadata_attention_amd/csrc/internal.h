// internal.h -- host-side types shared by the library's translation units.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "compilemask.h"
#include "preprocess_args.h"
#include "program.h"

struct cm_spec {
  cm::Program prog;              // lowered endpoint program, both directions
  int n_words = 0;
  int dir_off[2] = {2, 2};       // word offset of each direction
  int fixed_slots[2] = {0, 0};   // largest count of plain slots of a Region
  // per direction, per region: (plain slots, exists slots); K = max over regions
  std::vector<std::pair<int, int>> region_slots[2];
  std::vector<std::string> params;
  int n_refs = 0;
  uint64_t id = 0;               // unique per compiled spec
  std::string listing;           // human-readable lowered program
  // spec-specialised preprocess kernels (cm_spec_specialize), one per device
  struct Specialized {
    int device;
    void* module;                // hipModule_t
    void* function;              // hipFunction_t
  };
  std::vector<Specialized> specialized;
  mutable std::mutex specialized_mu;  // guards `specialized` (the rest never changes)
  ~cm_spec();
};

struct cm_desc {
  uint64_t spec_id = 0;
  int32_t B = 0, N = 0, seg_cap = 0, K_r = 0, K_c = 0;
  int32_t packed = 0;            // packed batch: number of samples (B is then 1)
  int32_t family = -1;           // block-mask descriptor of the predicate baseline: its family
  cm_metadata pred_md{};         // ... and the caller's metadata it refers to
  cm_tiles tiles{};
  int32_t Tq_f = 0, Tk_f = 0, Tk_b = 0, Tq_b = 0, Wf = 0, Wb = 0;
  size_t off[9] = {};            // section offsets + total (same order as cm_desc_offsets)
  void* buf = nullptr;
  size_t bytes = 0;
};

namespace cm {


// Thread-local error detail for cm_last_error().
void set_error(const std::string& msg);
cm_status fail(cm_status st, const std::string& msg);

// K of a direction for a segment capacity.
int spec_width(const cm_spec* spec, int dir, int seg_cap);

// Kernel launchers (HIP translation units).
hipError_t launch_preprocess(const PreprocessArgs& a, const Program& prog, hipStream_t stream);
size_t preprocess_lds_bytes(const PreprocessArgs& a);
// The spec-specialised kernel for the current device, or NULL.
void* specialized_function(const cm_spec* spec);
hipError_t launch_specialized(void* function, const PreprocessArgs& a, hipStream_t stream);
// HIP source of the spec-specialised preprocess kernel.
std::string specialized_source(const cm_spec* spec);
// Predicate baseline: per-token segment ids, then both tile bitmaps by
// evaluating the family's predicate at every element.
hipError_t launch_blockmask(const PreprocessArgs& a, int family, hipStream_t stream);

struct AttnDims {
  int32_t B, H, N, d;
  int64_t sb, sh, sn;            // element strides of the bf16 tensors
  float scale;
  int32_t causal;
  int32_t check;                 // partial-tile check, CM_CHECK_*
  int32_t precision;             // P / dS operand precision, CM_PRECISION_*
};
struct PredView {                // predicate-baseline inputs (block-mask descriptors)
  int32_t family;                 // -1: an interval descriptor
  const int32_t* tok_seg;
  const int32_t* scalars;
  int32_t n_scalars;
  const int32_t* refs;
  int32_t seg_cap, n_refs;
  const uint32_t* sample_err;
};
struct DescView {                // device pointers into a descriptor
  const uint32_t* fbm;
  const uint32_t* bbm;
  const uint32_t* row_iv;
  const uint32_t* col_iv;
  const uint32_t* row_tkmax;
  const uint32_t* col_tkmax;
  int32_t K_r, K_c, Wf, Wb, Tq_f, Tk_f, Tk_b, Tq_b;
  int32_t fq, fk, bk, bq;
  int32_t packed;                // packed batch: its sample count (0 for a padded batch or the causal path)
  PredView pred;
};
hipError_t launch_attn_fwd(const AttnDims& a, const void* q, const void* k, const void* v, const DescView& dv,
                           void* o, float* lse, hipStream_t stream);
// D[row] and lse2[row] (lse * log2(e), +inf for empty rows) into workspace
// D[0 .. B*H*N) and D[B*H*N .. 2*B*H*N)
hipError_t launch_bwd_dot(const AttnDims& a, const void* o, const void* dO, const float* lse, float* D,
                          hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnDims& a, const void* q, const void* k, const void* v, const float* lse,
                           const void* dO, const float* D, const DescView& dv, void* dk, void* dvv,
                           hipStream_t stream);
hipError_t launch_bwd_dq(const AttnDims& a, const void* q, const void* k, const void* v, const float* lse,
                         const void* dO, const float* D, const DescView& dv, void* dq, hipStream_t stream);
bool attn_tiles_supported(int d, int fq, int fk, int bk, int bq);
// dK/dV with 64 keys per wave (attn_dkdv_wide.hip): for 128-key backward
// tiles of 64 query rows, the default check and bf16 operands
bool dkdv_wide_supported(const AttnDims& a, const DescView& dv);
hipError_t launch_bwd_dkdv_wide(const AttnDims& a, const void* q, const void* k, const void* v, const void* dO,
                                const float* D, const DescView& dv, void* dk, void* dvv, hipStream_t stream);
// The fixed backward workspace of cm_attn_bwd_noalloc: 2 * kScratchRows floats
// per GPU; *ptr = its device address on the current device (looked up once
// per device).
constexpr size_t kScratchRows = size_t(CM_NOALLOC_MAX_ROWS);
hipError_t scratch_workspace(float** ptr);

}  // namespace cm
