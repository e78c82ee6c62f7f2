// Run-time compilation of the kernel source with hipRTC, one code object per
// KernelConfig, kept in memory and in an on-disk cache.
//
// DeepGEMM builds every kernel at run time with the shape as constants and
// keeps the results in a disk cache (launch article, section 4.2; README,
// utility functions and environment variables: DG_JIT_CACHE_DIR, DG_JIT_DEBUG,
// DG_JIT_PRINT_COMPILER_COMMAND).  Here the compiler is hipRTC targeting
// gfx950, and the cache directory is DG_CACHE_DIR (default: jit_cache/ next
// to libdg.so).  Files are named by a hash of (source, options, hipRTC
// version) and written through a temporary file and a rename, so a crash
// never leaves a truncated code object under a valid name.
#include <dlfcn.h>
#include <sys/stat.h>
#include <unistd.h>

#include <chrono>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>

#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include "dg_internal.h"

namespace dg {
namespace {

#include "kernel_source.inc"   // defines kKernelSource

std::mutex g_mu;
std::map<std::string, std::vector<char>> g_code;              // key -> code object
std::map<std::pair<int, std::string>, hipFunction_t> g_funcs;  // (device, key) -> function
std::vector<hipModule_t> g_modules;                           // kept until exit

uint64_t fnv1a(const void* data, size_t n, uint64_t h = 1469598103934665603ull) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

std::vector<std::string> compile_options(const KernelConfig& c) {
    std::vector<std::string> o = {
        "--offload-arch=gfx950", "-O3", "-std=c++20",
        // packed FP32 instructions stay off: the scalar forms are used throughout
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    };
    auto def = [&](const char* name, int v) { o.push_back(std::string("-D") + name + "=" + std::to_string(v)); };
    def("DG_KIND", c.kind);
    def("DG_BM", c.bm);
    def("DG_BN", c.bn);
    def("DG_WM", c.wm);
    def("DG_WN", c.wn);
    def("DG_STAGES", c.stages);
    def("DG_KSTEP", c.kstep);
    def("DG_SPLITK", c.splitk);
    def("DG_HAS_C", c.has_c);
    def("DG_N", c.n);
    def("DG_K", c.k);
    def("DG_G", c.g);
    def("DG_VARIANT", c.variant == 4 || c.variant == 6 ? 0 : c.variant);
    if (c.variant == 4) def("DG_AAHEAD", 1);
    if (c.variant == 6) def("DG_SPLIT", 1);
    def("DG_SF", c.sf);
    if (c.bstream) def("DG_BSTREAM", 1);
    if (c.ne > 0) {
        def("DG_NB", c.nb);
        def("DG_NE", c.ne);
    }
    return o;
}

std::string hex64(uint64_t v) {
    char buf[17];
    std::snprintf(buf, sizeof(buf), "%016llx", (unsigned long long)v);
    return buf;
}

// Identity of the hipRTC build in this process: its API version says little
// (different ROCm releases report the same one), so the loaded library's path
// and size go into the key too.
std::string compiler_identity() {
    int maj = 0, min = 0;
    hiprtcVersion(&maj, &min);
    std::string id = std::to_string(maj) + "." + std::to_string(min);
    Dl_info info;
    if (dladdr((void*)&hiprtcCompileProgram, &info) && info.dli_fname) {
        struct stat sb;
        id += std::string("|") + info.dli_fname;
        if (::stat(info.dli_fname, &sb) == 0) id += "|" + std::to_string((long long)sb.st_size);
    }
    return id;
}

std::string cache_file(const KernelConfig& c, const std::vector<std::string>& opts) {
    uint64_t h = fnv1a(kKernelSource, std::strlen(kKernelSource));
    for (const auto& s : opts) h = fnv1a(s.data(), s.size() + 1, h);
    const std::string id = compiler_identity();
    h = fnv1a(id.data(), id.size(), h);
    return cache_dir() + "/" + c.key() + "-" + hex64(h) + ".hsaco";
}

bool read_file(const std::string& path, std::vector<char>* out) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    std::vector<char> buf((std::istreambuf_iterator<char>(f)), std::istreambuf_iterator<char>());
    // a code object is an ELF file: reject anything else (e.g. a damaged cache entry)
    if (buf.size() < 64 || std::memcmp(buf.data(), "\x7f" "ELF", 4) != 0) return false;
    *out = std::move(buf);
    return true;
}

void write_file_atomic(const std::string& path, const std::vector<char>& data) {
    std::string dir = cache_dir();
    ::mkdir(dir.c_str(), 0755);
    std::string tmp = path + ".tmp" + std::to_string(::getpid());
    {
        std::ofstream f(tmp, std::ios::binary);
        if (!f) return;                      // unwritable directory: memory cache only
        f.write(data.data(), (std::streamsize)data.size());
        if (!f) {
            ::unlink(tmp.c_str());
            return;
        }
    }
    if (std::rename(tmp.c_str(), path.c_str()) != 0) ::unlink(tmp.c_str());
}

dg_status compile_locked(const KernelConfig& c, std::vector<char>* code) {
    std::vector<std::string> opts = compile_options(c);
    // the extra option changes the code, so it is part of both cache keys
    const std::string extra = jit_extra_option();
    if (!extra.empty()) opts.push_back(extra);
    const std::string mem_key = c.key() + (extra.empty() ? std::string() : "|" + extra);
    auto it = g_code.find(mem_key);
    if (it != g_code.end()) {
        *code = it->second;
        return DG_OK;
    }
    const std::string path = cache_file(c, opts);
    if (read_file(path, code)) {
        g_code[mem_key] = *code;
        return DG_OK;
    }
    const bool verbose = env_flag("DG_PRINT_COMPILE");
    auto t0 = std::chrono::steady_clock::now();
    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, kKernelSource, "fp8_gemm.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS)
        return set_error(DG_ERR_JIT, "hiprtcCreateProgram failed");
    std::vector<const char*> argv;
    for (const auto& s : opts) argv.push_back(s.c_str());
    hiprtcResult r = hiprtcCompileProgram(prog, (int)argv.size(), argv.data());
    size_t log_size = 0;
    hiprtcGetProgramLogSize(prog, &log_size);
    std::string log(log_size, '\0');
    if (log_size) hiprtcGetProgramLog(prog, &log[0]);
    if (r != HIPRTC_SUCCESS) {
        hiprtcDestroyProgram(&prog);
        return set_error(DG_ERR_JIT, "hipRTC compile of " + c.key() + " failed: " + log);
    }
    size_t size = 0;
    hiprtcGetCodeSize(prog, &size);
    code->assign(size, 0);
    hiprtcGetCode(prog, code->data());
    hiprtcDestroyProgram(&prog);
    if (verbose) {
        double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        std::ostringstream cmd;
        for (const auto& s : opts) cmd << ' ' << s;
        std::fprintf(stderr, "[dg] hipRTC %s (%.0f ms):%s\n", c.key().c_str(), ms, cmd.str().c_str());
    }
    g_code[mem_key] = *code;
    write_file_atomic(path, *code);
    return DG_OK;
}

}  // namespace

std::string KernelConfig::key() const {
    std::ostringstream s;
    s << "k" << kind << (variant ? "v" + std::to_string(variant) : std::string()) << "_m" << bm << "n" << bn << "_w" << wm << "x" << wn << "_s" << stages << "x" << kstep
      << "_sk" << splitk
      << "_c" << has_c << "_N" << n << "_K" << k << "_G" << g;
    if (bstream) s << "_bs";
    if (sf == 1) s << "_e8m0";
    if (sf == 2) s << "_f8f4";
    if (sf == 3) s << "_bf16";
    if (sf == 4) s << "_f4f4";
    if (sf == 5) s << "_e8m0x2";
    if (ne > 0) s << "_cols" << nb << "-" << ne;
    return s.str();
}

std::string cache_dir() {
    const char* env = std::getenv("DG_CACHE_DIR");
    if (env && *env) return env;
    Dl_info info;
    if (dladdr((void*)&cache_dir, &info) && info.dli_fname) {
        std::string so = info.dli_fname;
        auto pos = so.rfind('/');
        if (pos != std::string::npos) return so.substr(0, pos) + "/jit_cache";
    }
    return "jit_cache";
}

// One more hipRTC option from the environment: tests force a compile error with
// it, experiments pass -D switches.  A build with it is never served to a caller
// without it (or with another): the option is part of every cache key.
std::string jit_extra_option() {
    const char* v = std::getenv("DG_JIT_EXTRA_OPTION");
    return v ? std::string(v) : std::string();
}

// Largest value of a code-object metadata field (a msgpack string key followed
// by an unsigned integer) over the kernels of the object; 0 if absent.
uint64_t metadata_max(const std::vector<char>& code, const std::string& key) {
    uint64_t best = 0;
    const std::string k = key;
    for (size_t pos = 0; (pos = std::string(code.data(), code.size()).find(k, pos)) != std::string::npos; pos += k.size()) {
        size_t i = pos + k.size();
        if (i >= code.size()) break;
        const unsigned char t = (unsigned char)code[i];
        uint64_t v = 0;
        if (t <= 0x7f) v = t;                                       // positive fixint
        else if (t >= 0xcc && t <= 0xcf) {                          // uint 8/16/32/64, big-endian
            const int n = 1 << (t - 0xcc);
            if (i + n >= code.size()) break;
            for (int b = 1; b <= n; ++b) v = (v << 8) | (unsigned char)code[i + b];
        }
        best = std::max(best, v);
    }
    return best;
}

// The variants that load B straight into VGPRs (1, 2, 3, 5) keep loads in flight
// into registers the compiler believes written at issue; a spill there could
// hand such a register to another value while the load is still landing.  Their
// code objects must therefore use no scratch at all.
dg_status check_register_loads(const KernelConfig& c, const std::vector<char>& code) {
    if (c.variant == 0 || c.variant == 4 || c.variant == 6) return DG_OK;
    const uint64_t scratch = metadata_max(code, ".private_segment_fixed_size");
    const uint64_t spills = metadata_max(code, ".vgpr_spill_count");
    if (scratch || spills)
        return set_error(DG_ERR_JIT, c.key() + ": this kernel variant must not spill registers (" +
                                         std::to_string(spills) + " VGPRs spilled, " + std::to_string(scratch) +
                                         " bytes of scratch); pick a smaller tile");
    return DG_OK;
}

dg_status compile_code(const KernelConfig& c, std::vector<char>* code) {
    std::lock_guard<std::mutex> lock(g_mu);
    dg_status s = compile_locked(c, code);
    return s != DG_OK ? s : check_register_loads(c, *code);
}

dg_status get_function(const KernelConfig& c, void** function, const char* name) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return set_error(DG_ERR_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_mu);
    const std::string extra = jit_extra_option();
    auto key = std::make_pair(dev, c.key() + "/" + name + (extra.empty() ? std::string() : "|" + extra));
    auto it = g_funcs.find(key);
    if (it != g_funcs.end()) {
        *function = (void*)it->second;
        return DG_OK;
    }
    std::vector<char> code;
    dg_status s = compile_locked(c, &code);
    if (s != DG_OK) return s;
    s = check_register_loads(c, code);
    if (s != DG_OK) return s;
    auto t0 = std::chrono::steady_clock::now();
    hipModule_t mod;
    hipError_t e = hipModuleLoadData(&mod, code.data());
    if (e != hipSuccess)
        return set_error(DG_ERR_JIT, std::string("hipModuleLoadData failed: ") + hipGetErrorString(e));
    hipFunction_t f;
    e = hipModuleGetFunction(&f, mod, name);
    if (e != hipSuccess)
        return set_error(DG_ERR_JIT, std::string("hipModuleGetFunction failed: ") + hipGetErrorString(e));
    if (env_flag("DG_PRINT_COMPILE")) {
        double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        std::fprintf(stderr, "[dg] loaded %s on device %d (%.1f ms)\n", c.key().c_str(), dev, ms);
    }
    g_modules.push_back(mod);
    g_funcs[key] = f;
    *function = (void*)f;
    return DG_OK;
}

}  // namespace dg
