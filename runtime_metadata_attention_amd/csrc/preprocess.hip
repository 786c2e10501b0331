// preprocess.hip -- online preprocess: batch metadata -> Execution Descriptor.
//
// CompileMask paper summary, section 3.3 "Online Efficient Mask Attention
// Execution": the preprocess kernel evaluates the compiled endpoints against
// the batch metadata and builds the descriptors of the forward and backward
// passes; section 3.3.1 "Execution Descriptor": an Interval Table padded with
// zero-length intervals, and two-bit tile states (empty / full / partial).
//
// One launch builds everything.  Grid (Tq_f + Tk_b, B): work-group x < Tq_f
// owns forward query tile x (its rows' key runs, its forward bitmap row and
// run maximum); the others own one backward key tile (its columns' row runs,
// its backward bitmap row and run maximum).  No work-group reads another's
// output, so there are no global atomics and no memset; every byte of the
// variable sections is rewritten on every build.
//
// Packed batches (B = 1, one sequence of N tokens made of n_samples samples
// laid end to end): each index finds its sample in cu_seqlens, evaluates the
// rules in the sample's coordinates (its length plays the part of N) and
// shifts the runs by the sample's first token, so no run leaves its sample.
//
// Tile states come from two counters per tile of the other axis, kept as
// difference arrays in LDS: `any` (how many of the work-group's indices have a
// run touching the tile) and `full` (how many have the whole tile inside one
// run).  A prefix scan turns them into counts: any == 0 -> empty, full == the
// number of indices -> full, otherwise partial.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "preprocess_core.h"

namespace cm {
namespace {

// Both structs travel in one kernel argument.  The kernel reads them through
// the kernarg segment pointer (explicit arguments start at offset 0 of that
// segment), so that the program, which is indexed with run-time offsets, is
// read in place with scalar loads instead of being copied to private memory.
struct KernArgs {
  PreprocessArgs a;
  Program prog;
};

__global__ __launch_bounds__(pre::kThreads) void preprocess_kernel(KernArgs /*in kernarg segment*/) {
#if defined(__HIP_DEVICE_COMPILE__)
  const KernArgs* ka = (const KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  pre::preprocess_body(ka->a, ka->prog.w);
#endif
}

}  // namespace

size_t preprocess_lds_bytes(const PreprocessArgs& a) { return sizeof(int32_t) * size_t(preprocess_lds_words(a)); }

hipError_t launch_preprocess(const PreprocessArgs& a, const Program& prog, hipStream_t stream) {
  dim3 grid(a.Tq_f + a.Tk_b, a.B);
  KernArgs ka;
  ka.a = a;
  ka.prog = prog;
  hipLaunchKernelGGL(preprocess_kernel, grid, dim3(pre::kThreads), preprocess_lds_bytes(a), stream, ka);
  return hipGetLastError();
}

}  // namespace cm
