// oeq_jitc: compiles one plan's generated HIP source to a gfx950 code object with the
// ROCm installation this library was built against.
//
//   oeq_jitc SOURCE_FILE OUTPUT_FILE      (exit status 0 on success)
//
// liboeq.so runs it as a child process.  The runtime compiler loads its compiler
// library (amd_comgr, which contains LLVM) by soname, so inside a process that has
// already loaded another ROCm release's copy (a framework wheel that bundles its own
// ROCm libraries) it would silently compile with that release's LLVM, whose code for
// these kernels is slower.  Here, in a fresh process, the compiler library is loaded
// by absolute path from the directory of the runtime compiler itself before the first
// compile, so every plan is compiled by the same release.
#include <dlfcn.h>

#include <cstdio>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include <hip/hiprtc.h>

#include "jit_options.hpp"

int main(int argc, char **argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: oeq_jitc SOURCE_FILE OUTPUT_FILE\n");
        return 2;
    }
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&hiprtcCompileProgram), &info) && info.dli_fname) {
        std::string dir = info.dli_fname;
        const auto pos = dir.find_last_of('/');
        if (pos != std::string::npos) {
            const std::string comgr = dir.substr(0, pos) + "/libamd_comgr.so.3";
            (void)dlopen(comgr.c_str(), RTLD_NOW | RTLD_GLOBAL);  // the runtime compiler then finds it loaded
        }
    }
    std::ifstream in(argv[1], std::ios::binary);
    if (!in) {
        std::fprintf(stderr, "oeq_jitc: cannot read %s\n", argv[1]);
        return 1;
    }
    std::stringstream ss;
    ss << in.rdbuf();
    const std::string src = ss.str();
    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, src.c_str(), "oeq_tp_conv.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
        std::fprintf(stderr, "oeq_jitc: hiprtcCreateProgram failed\n");
        return 1;
    }
    const hiprtcResult rc = hiprtcCompileProgram(prog, oeq::kJitOptionCount, oeq::kJitOptions);
    if (rc != HIPRTC_SUCCESS) {
        size_t n = 0;
        hiprtcGetProgramLogSize(prog, &n);
        std::string log(n + 1, '\0');
        if (n) hiprtcGetProgramLog(prog, &log[0]);
        std::fprintf(stderr, "oeq_jitc: compile failed: %s\n%s\n", hiprtcGetErrorString(rc), log.c_str());
        hiprtcDestroyProgram(&prog);
        return 1;
    }
    size_t size = 0;
    hiprtcGetCodeSize(prog, &size);
    std::vector<char> code(size);
    hiprtcGetCode(prog, code.data());
    hiprtcDestroyProgram(&prog);
    std::ofstream out(argv[2], std::ios::binary);
    out.write(code.data(), static_cast<std::streamsize>(code.size()));
    if (!out) {
        std::fprintf(stderr, "oeq_jitc: cannot write %s\n", argv[2]);
        return 1;
    }
    return 0;
}
