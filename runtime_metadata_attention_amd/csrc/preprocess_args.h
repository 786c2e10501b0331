// preprocess_args.h -- what the preprocess kernel receives (plain data, no
// host API), shared by the library and the run-time compiled, spec-specialised
// preprocess kernel.
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

namespace cm {

// Descriptor sections, in layout order (cm_desc_offsets).
enum Section { SEC_HEADER = 0, SEC_SAMPLE_ERR, SEC_ROW_TKMAX, SEC_COL_TKMAX, SEC_FBM, SEC_BBM,
               SEC_ROW_IV, SEC_COL_IV, SEC_TOTAL };

// Same values as CM_DESC_MAGIC and CM_MD_CU_SEQLENS (include/compilemask.h).
constexpr uint32_t kDescMagic = 0x31444D43u;
constexpr uint32_t kMdCuSeqlens = 16u;

struct PreprocessArgs {
  const int32_t* scalars;
  const int32_t* seg_bounds;
  const int32_t* n_seg;
  const int32_t* refs;
  const int32_t* cu_seqlens;      // packed batch: [n_samples + 1], else NULL
  int32_t n_samples;              // packed batch: samples (metadata rows), else 0
  int32_t n_scalars, n_refs, seg_cap;
  uint32_t* desc;                 // descriptor base
  int32_t B, N, K_r, K_c;
  int32_t fq, fk, bk, bq;         // tile sizes
  int32_t Tq_f, Tk_f, Tk_b, Tq_b, Wf, Wb;
  uint32_t off_words[8];          // section offsets in words
  int32_t dir_off[2];
};

// Threads per work-group and dynamic LDS words of the preprocess kernel.
constexpr int kPreThreads = 256;
inline
#ifdef __HIPCC__
__host__ __device__
#endif
int preprocess_lds_words(const PreprocessArgs& a) {
  const int Tmax = a.Tk_f > a.Tq_b ? a.Tk_f : a.Tq_b;
  return 2 * (Tmax + 1) + 2 * kPreThreads + 4 + (a.seg_cap + 1) + a.seg_cap * a.n_refs + a.n_scalars;
}

}  // namespace cm
