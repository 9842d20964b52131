// Options of the runtime compile of a plan's kernels (shared by the library and the
// compiler helper, so both compile exactly the same way).
#pragma once

namespace oeq {

inline const char *const kJitOptions[] = {
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-munsafe-fp-atomics",
    // packed fp32 instructions are kept out of all generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};
constexpr int kJitOptionCount = static_cast<int>(sizeof(kJitOptions) / sizeof(kJitOptions[0]));

}  // namespace oeq
