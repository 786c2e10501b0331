// specialize.cpp -- spec-specialised preprocess kernels, compiled at run time.
//
// The CompileMask paper summary (sections 1 and 3.1) compiles each MaskSpec
// once and then preprocesses every batch with the compiled result.  The
// library's default preprocess interprets the lowered endpoint program; this
// file generates a kernel in which the program is a compile-time constant
// array, compiles it with hipRTC for gfx950 and loads it.  The kernel body is
// the same code (preprocess_core.h, embedded in the library at build time),
// so the compiler folds the program walk into straight-line endpoint
// arithmetic and the descriptor is bit-identical.
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <string>
#include <vector>

#include "internal.h"

namespace cm {

// Filled by the build (csrc/*.h embedded as strings).
extern const int kRtcHeaderCount;
extern const char* const kRtcHeaderNames[];
extern const char* const kRtcHeaderSources[];

std::string specialized_source(const cm_spec* spec) {
  std::string s;
  s += "// spec-specialised preprocess kernel (generated)\n";
  s += "#include \"preprocess_core.h\"\n\n";
  s += "__device__ constexpr int32_t kProgram[" + std::to_string(spec->n_words) + "] = {";
  for (int i = 0; i < spec->n_words; ++i) s += (i ? ", " : "") + std::to_string(spec->prog.w[i]);
  s += "};\n\n";
  s += "extern \"C\" __global__ __launch_bounds__(256) void cm_preprocess_specialized(cm::PreprocessArgs a) {\n";
  s += "  cm::pre::preprocess_body(a, kProgram);\n}\n";
  return s;
}

static void* find_specialized(const cm_spec* spec, int dev) {
  for (const auto& x : spec->specialized)
    if (x.device == dev) return x.function;
  return nullptr;
}

void* specialized_function(const cm_spec* spec) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(spec->specialized_mu);
  return find_specialized(spec, dev);
}

hipError_t launch_specialized(void* function, const PreprocessArgs& a, hipStream_t stream) {
  PreprocessArgs arg = a;
  void* params[] = {&arg};
  return hipModuleLaunchKernel(static_cast<hipFunction_t>(function), unsigned(a.Tq_f + a.Tk_b), unsigned(a.B), 1,
                               unsigned(kPreThreads), 1, 1, unsigned(preprocess_lds_bytes(a)), stream, params, nullptr);
}

}  // namespace cm

cm_spec::~cm_spec() {
  int cur = -1;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (const auto& x : specialized) {
    if (hipSetDevice(x.device) == hipSuccess) (void)hipModuleUnload(static_cast<hipModule_t>(x.module));
  }
  if (have) (void)hipSetDevice(cur);
}

using namespace cm;

extern "C" {

cm_status cm_spec_codegen(const cm_spec* spec, char* buf, size_t len, size_t* needed) {
  if (!spec) return fail(CM_ERR_NULL, "spec is NULL");
  const std::string s = specialized_source(spec);
  if (needed) *needed = s.size() + 1;
  if (buf && len) {
    const size_t n = s.size() < len - 1 ? s.size() : len - 1;
    for (size_t i = 0; i < n; ++i) buf[i] = s[i];
    buf[n] = 0;
  }
  return CM_OK;
}

cm_status cm_spec_specialize(cm_spec* spec) {
  if (!spec) return fail(CM_ERR_NULL, "spec is NULL");
  int dev = -1;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return fail(CM_ERR_HIP, std::string("cm_spec_specialize: ") + hipGetErrorString(he));
  if (specialized_function(spec)) return CM_OK;
  // compiled without the lock (about a second); a second caller that raced
  // this one for the same device keeps the first module and drops its own
  const std::string src = specialized_source(spec);
  hiprtcProgram prog;
  hiprtcResult r = hiprtcCreateProgram(&prog, src.c_str(), "cm_preprocess_specialized.hip", kRtcHeaderCount,
                                       kRtcHeaderSources, kRtcHeaderNames);
  if (r != HIPRTC_SUCCESS) return fail(CM_ERR_HIP, std::string("hiprtcCreateProgram: ") + hiprtcGetErrorString(r));
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
  r = hiprtcCompileProgram(prog, int(sizeof(opts) / sizeof(opts[0])), opts);
  if (r != HIPRTC_SUCCESS) {
    size_t n = 0;
    hiprtcGetProgramLogSize(prog, &n);
    std::string log(n, '\0');
    if (n) hiprtcGetProgramLog(prog, &log[0]);
    hiprtcDestroyProgram(&prog);
    return fail(CM_ERR_HIP, std::string("hiprtcCompileProgram: ") + hiprtcGetErrorString(r) + "\n" + log);
  }
  size_t code_size = 0;
  hiprtcGetCodeSize(prog, &code_size);
  std::vector<char> code(code_size);
  hiprtcGetCode(prog, code.data());
  hiprtcDestroyProgram(&prog);
  hipModule_t module;
  he = hipModuleLoadData(&module, code.data());
  if (he != hipSuccess) return fail(CM_ERR_HIP, std::string("hipModuleLoadData: ") + hipGetErrorString(he));
  hipFunction_t function;
  he = hipModuleGetFunction(&function, module, "cm_preprocess_specialized");
  if (he != hipSuccess) {
    (void)hipModuleUnload(module);
    return fail(CM_ERR_HIP, std::string("hipModuleGetFunction: ") + hipGetErrorString(he));
  }
  {
    std::lock_guard<std::mutex> lock(spec->specialized_mu);
    if (!find_specialized(spec, dev)) {
      spec->specialized.push_back({dev, module, function});
      return CM_OK;
    }
  }
  (void)hipModuleUnload(module);
  return CM_OK;
}

}  // extern "C"
