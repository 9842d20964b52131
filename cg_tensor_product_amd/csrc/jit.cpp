// Runtime compilation of a plan's kernels with hipRTC for gfx950, an on-disk
// code-object cache keyed by a hash of the generated source and the options, and
// per-device module loading.
//
// The compile runs in the helper program oeq_jitc beside this library (a child
// process): in a process that has loaded another ROCm release's compiler library
// first, an in-process compile would use that release's LLVM (see jitc_main.cpp).
// OEQ_JIT_IN_PROCESS=1, or a missing or failing helper, compiles here instead.
//
// Compiling the path-specialised kernels when the plan is made mirrors the
// runtime template selection discussed in "Receiver-streaming convolutions for
// channel-wise UVU tensor products" (maintainer replies) and the compile-time
// static analysis of "An Efficient Sparse Kernel Generator ..." (abstract).
#include <dlfcn.h>
#include <spawn.h>
#include <sys/stat.h>
#include <sys/wait.h>
#include <unistd.h>

#include <atomic>

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include <hip/hiprtc.h>

#include "jit_options.hpp"
#include "planner.hpp"

extern char **environ;

namespace oeq {

namespace {

const char *const *const kOptions = kJitOptions;

uint64_t fnv1a(const std::string &s, uint64_t h = 1469598103934665603ULL) {
    for (unsigned char c : s) {
        h ^= c;
        h *= 1099511628211ULL;
    }
    return h;
}

// Directory of this library.
std::string lib_dir() {
    Dl_info info;
    if (dladdr(reinterpret_cast<void *>(&lib_dir), &info) && info.dli_fname) {
        std::string f = info.dli_fname;
        const auto pos = f.find_last_of('/');
        if (pos != std::string::npos) return f.substr(0, pos);
    }
    return "";
}

std::string cache_dir() {
    if (const char *e = std::getenv("OEQ_CACHE_DIR")) return e;
    const std::string d = lib_dir();
    return d.empty() ? d : d + "/jitcache";
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

// Compiles p.source with the helper program into p.code.  Returns false (p.code untouched)
// when the helper is missing or fails; `dir` is a writable directory for the two files
// passed to it.
bool compile_in_helper(oeq_plan &p, const std::string &dir, std::string *why) {
    static std::atomic<int> counter{0};
    const std::string helper = lib_dir() + "/oeq_jitc";
    if (access(helper.c_str(), X_OK) != 0) {
        if (why) *why = "compiler helper " + helper + " not found";
        return false;
    }
    const std::string stem = dir + "/" + p.code_key + "." + std::to_string(static_cast<long>(getpid())) + "." +
                             std::to_string(counter++);
    const std::string src = stem + ".hip", out = stem + ".co";
    {
        std::ofstream f(src, std::ios::binary);
        f << p.source;
        if (!f) {
            if (why) *why = "cannot write " + src;
            return false;
        }
    }
    char *argv[] = {const_cast<char *>(helper.c_str()), const_cast<char *>(src.c_str()),
                    const_cast<char *>(out.c_str()), nullptr};
    pid_t pid = 0;
    int status = -1;
    const int e = posix_spawn(&pid, helper.c_str(), nullptr, nullptr, argv, environ);
    bool ok = e == 0 && waitpid(pid, &status, 0) == pid && WIFEXITED(status) && WEXITSTATUS(status) == 0;
    std::vector<char> code;
    ok = ok && read_file(out, code);
    std::remove(src.c_str());
    std::remove(out.c_str());
    if (!ok) {
        if (why) *why = "compiler helper failed (status " + std::to_string(status) + ")";
        return false;
    }
    p.code.swap(code);
    return true;
}

}  // namespace

oeq_status jit_compile(oeq_plan &p, std::string *why, bool cache_only) {
    int ver_major = 0, ver_minor = 0;
    hiprtcVersion(&ver_major, &ver_minor);
    std::ostringstream key;
    key << p.source << '\n' << ver_major << '.' << ver_minor;
    for (int i = 0; i < kJitOptionCount; ++i) key << ' ' << kOptions[i];
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
    if (!std::getenv("OEQ_JIT_IN_PROCESS")) {
        std::string hdir = use_cache ? dir : "";
        if (use_cache) mkdir(dir.c_str(), 0775);
        if (hdir.empty() || access(hdir.c_str(), W_OK) != 0) {
            const char *t = std::getenv("TMPDIR");
            hdir = t && *t ? t : "/tmp";
        }
        std::string hwhy;
        if (compile_in_helper(p, hdir, &hwhy)) {
            if (std::getenv("OEQ_LOG"))
                std::fprintf(stderr, "[oeq] compiled %s in the helper (%zu bytes)\n", p.code_key.c_str(), p.code.size());
            if (use_cache) write_file_atomic(path, p.code);
            return OEQ_OK;
        }
        if (std::getenv("OEQ_LOG")) std::fprintf(stderr, "[oeq] %s; compiling in this process\n", hwhy.c_str());
    }

    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, p.source.c_str(), "oeq_tp_conv.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS) {
        if (why) *why = "hiprtcCreateProgram failed";
        return OEQ_ERR_JIT;
    }
    const int nopt = kJitOptionCount;
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
