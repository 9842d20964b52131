// Runtime compilation of a plan's kernels with hipRTC for gfx950, an on-disk
// code-object cache keyed by a hash of the generated source and the options, and
// per-device module loading.
//
// Compiling the path-specialised kernels when the plan is made mirrors the
// runtime template selection discussed in "Receiver-streaming convolutions for
// channel-wise UVU tensor products" (maintainer replies) and the compile-time
// static analysis of "An Efficient Sparse Kernel Generator ..." (abstract).
#include <dlfcn.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include <hip/hiprtc.h>

#include "planner.hpp"

namespace oeq {

namespace {

const char *const kOptions[] = {
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-munsafe-fp-atomics",
    // packed fp32 instructions are kept out of all generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};

uint64_t fnv1a(const std::string &s, uint64_t h = 1469598103934665603ULL) {
    for (unsigned char c : s) {
        h ^= c;
        h *= 1099511628211ULL;
    }
    return h;
}

std::string cache_dir() {
    if (const char *e = std::getenv("OEQ_CACHE_DIR")) return e;
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&cache_dir), &info) && info.dli_fname) {
        std::string f = info.dli_fname;
        const auto pos = f.find_last_of('/');
        if (pos != std::string::npos) return f.substr(0, pos) + "/jitcache";
    }
    return "";
}

bool read_file(const std::string &path, std::vector<char> &out) {
    std::ifstream in(path, std::ios::binary);
    if (!in) return false;
    in.seekg(0, std::ios::end);
    const std::streamoff n = in.tellg();
    if (n <= 0) return false;
    out.resize(static_cast<size_t>(n));
    in.seekg(0);
    in.read(out.data(), n);
    return static_cast<bool>(in);
}

void write_file_atomic(const std::string &path, const std::vector<char> &data) {
    const std::string tmp = path + ".tmp" + std::to_string(static_cast<long>(getpid()));
    {
        std::ofstream out(tmp, std::ios::binary);
        if (!out) return;
        out.write(data.data(), static_cast<std::streamsize>(data.size()));
        if (!out) {
            std::remove(tmp.c_str());
            return;
        }
    }
    if (std::rename(tmp.c_str(), path.c_str()) != 0) std::remove(tmp.c_str());
}

}  // namespace

oeq_status jit_compile(oeq_plan &p, std::string *why, bool cache_only) {
    int ver_major = 0, ver_minor = 0;
    hiprtcVersion(&ver_major, &ver_minor);
    std::ostringstream key;
    key << p.source << '\n' << ver_major << '.' << ver_minor;
    for (const char *o : kOptions) key << ' ' << o;
    char hex[32];
    std::snprintf(hex, sizeof hex, "%016llx", static_cast<unsigned long long>(fnv1a(key.str())));
    p.code_key = hex;

    const std::string dir = cache_dir();
    const bool use_cache = !dir.empty() && std::getenv("OEQ_NO_CACHE") == nullptr;
    const std::string path = dir + "/" + p.code_key + ".hsaco";
    if (std::getenv("OEQ_DUMP_SOURCE") && !dir.empty()) {
        mkdir(dir.c_str(), 0775);
        std::ofstream(dir + "/" + p.code_key + ".hip") << p.source;
    }
    if (use_cache && read_file(path, p.code)) return OEQ_OK;
    if (cache_only) {
        if (why) *why = "code object " + p.code_key + " is not in the cache";
        return OEQ_ERR_JIT;
    }

    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, p.source.c_str(), "oeq_tp_conv.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
        if (why) *why = "hiprtcCreateProgram failed";
        return OEQ_ERR_JIT;
    }
    const int nopt = static_cast<int>(sizeof(kOptions) / sizeof(kOptions[0]));
    const hiprtcResult rc = hiprtcCompileProgram(prog, nopt, kOptions);
    size_t log_size = 0;
    hiprtcGetProgramLogSize(prog, &log_size);
    std::string log(log_size + 1, '\0');
    if (log_size) hiprtcGetProgramLog(prog, &log[0]);
    if (rc != HIPRTC_SUCCESS) {
        if (why) *why = std::string("hipRTC compile failed: ") + hiprtcGetErrorString(rc) + "\n" + log;
        hiprtcDestroyProgram(&prog);
        return OEQ_ERR_JIT;
    }
    size_t code_size = 0;
    hiprtcGetCodeSize(prog, &code_size);
    p.code.resize(code_size);
    hiprtcGetCode(prog, p.code.data());
    hiprtcDestroyProgram(&prog);
    if (std::getenv("OEQ_LOG")) std::fprintf(stderr, "[oeq] compiled %s (%zu bytes)\n%s", p.code_key.c_str(), code_size, log.c_str());
    if (use_cache) {
        mkdir(dir.c_str(), 0775);
        write_file_atomic(path, p.code);
    }
    return OEQ_OK;
}

bool module_loaded(oeq_plan &p, int dev) {
    std::lock_guard<std::mutex> lock(p.mu);
    const auto it = p.modules.find(dev);
    return it != p.modules.end() && it->second.module != nullptr;
}

oeq_status get_kernel(oeq_plan &p, const char *name, hipFunction_t *fn, std::string *why) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        if (why) *why = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return OEQ_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(p.mu);
    DeviceModule &dm = p.modules[dev];
    if (!dm.module) {
        e = hipModuleLoadData(&dm.module, p.code.data());
        if (e != hipSuccess) {
            dm.module = nullptr;
            if (why) *why = std::string("hipModuleLoadData: ") + hipGetErrorString(e);
            return OEQ_ERR_HIP;
        }
    }
    auto it = dm.fn.find(name);
    if (it != dm.fn.end()) {
        *fn = it->second;
        return OEQ_OK;
    }
    hipFunction_t f = nullptr;
    e = hipModuleGetFunction(&f, dm.module, name);
    if (e != hipSuccess) {
        if (why) *why = std::string("hipModuleGetFunction(") + name + "): " + hipGetErrorString(e);
        return OEQ_ERR_HIP;
    }
    dm.fn[name] = f;
    *fn = f;
    return OEQ_OK;
}

}  // namespace oeq
