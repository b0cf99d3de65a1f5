// proj.cpp -- the C ABI of libproj (declared in include/proj.h): argument
// checks, the per-context workspace, the measured plan cache and HIP-graph
// capture of repeated calls.
//
// Plan choice follows the rule that a method wins only at a given size and
// that the choice is made by measuring, not by thresholds fitted to one
// machine (worklog "How I made Muse's GPU projections 1.32x faster in the
// Open Kernel Challenge", section "I started picking a method based on the
// job"; page "blackroom" on Devpost, sections "How we built it" and "What we
// learned"): on the first uncaptured call for a shape, every compiled kernel
// variant valid for the shape is timed on the caller's buffers and the
// fastest is kept.  Under stream capture nothing may be timed or
// synchronised, so an untimed default plan is used until a later uncaptured
// tune.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/proj.h"
#include "kernels.hpp"

using namespace proj;

// Split-K partials of proj_run_noalloc live in this file-scope device array
// instead of a context's workspace, so that call allocates nothing.  In host
// code the array's name is only a stand-in: its device address is resolved
// once per device with hipGetSymbolAddress (with that device current, when a
// context is created on it), and only that address is passed to kernels.
// Every call on one GPU shares that GPU's copy, which keeps the last call's
// contents; nothing in it needs to start at zero (a split plan rewrites all
// of its partials before summing them).
static constexpr size_t kScratchBytes = size_t{2} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr uint32_t kMagic = 0x50524f4au;   // live context
constexpr uint32_t kDead = 0xdeadbeefu;    // destroyed context
constexpr size_t kZeroBytes = 256;   // zero page for masked loads
constexpr size_t kSinkBytes = 1024;  // target of the read kernels' never-taken store
constexpr size_t kFlushBytes = 512ull << 20;  // larger than the last-level cache

// K is the depth of the product: for a hi/lo weight pair (hilo = 1) twice
// the X row length
struct Key {
    int64_t M, N, K;
    int epi, out, aligned;
    int hilo = 0;
    int wpack = 0;  // packed weights: 16-row units per tile (0: row-major W)
    bool operator<(const Key &o) const {
        return std::tie(M, N, K, epi, out, aligned, hilo, wpack) <
               std::tie(o.M, o.N, o.K, o.epi, o.out, o.aligned, o.hilo, o.wpack);
    }
};

enum Kind { KIND_STREAM = 0, KIND_GEMM = 1, KIND_GENERIC = 2, KIND_GEMV = 3 };

struct Candidate {
    Kind kind;
    int variant;  // index into the kernel table
    int splits;   // K ranges over workgroups (1: no split)
    std::string name;
    int atomic = 0;  // splits added into a zeroed fp32 Y with atomics instead of a workspace pass
    int walk = 0;    // streaming kernel's K-walk stride (Args::walk; 0: 7)
};

struct Plan {
    Candidate cand;
    bool tuned;
    float us;  // measured median (tuned plans)
};

}  // namespace

struct proj_ctx {
    uint32_t magic;
    int device;
    void *scratch_dev;   // device address of this device's copy of `scratch`
    int cus;             // compute units of the device
    double cu_flops;     // one CU's dense bf16 matrix rate (flop/s) at the device clock
    float *ws;           // split-K partial workspace, ws_bytes long (caller-bounded)
    size_t ws_bytes;
    uint16_t *zeros;     // kZeroBytes of zeros, then kSinkBytes of sink (one allocation)
    std::map<Key, Plan> plans;
    std::mutex mu;
    std::string err;
    std::string dev_id;  // architecture and CU count: the plan file's device key
};

// A captured graph keeps the context's workspace and zero page as kernel
// arguments, so it remembers its context: once that is destroyed the graph
// is not replayed.
struct proj_graph {
    uint32_t magic;
    int device;
    proj_ctx *ctx;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

namespace {

bool env_flag(const char *name, bool dflt);

// ---- optional plan file and log.  PROJ_PLAN_FILE names a text file of
// measured plans: each tuned plan is appended as one line
//   proj-plan 1 <device> <M> <N> <K> <epi> <out> <aligned> <hilo> <wpack> <plan> <us>
// and proj_create loads the lines of its device (architecture and CU
// count), the last line of a key winning, so a later process or context
// starts from the measured plans instead of tuning again.  A line whose plan
// is not a candidate of its key (another library build), or whose partials
// do not fit the context's workspace, is skipped.  PROJ_LOG=1 prints each
// plan decision to stderr.
bool plan_log() { return env_flag("PROJ_LOG", false); }

void save_plan(const proj_ctx *c, const Key &k, const Plan &p) {
    const char *path = std::getenv("PROJ_PLAN_FILE");
    if (!path || !*path) return;
    FILE *f = std::fopen(path, "a");
    if (!f) return;
    std::fprintf(f, "proj-plan 1 %s %lld %lld %lld %d %d %d %d %d %s %.3f\n", c->dev_id.c_str(), (long long)k.M,
                 (long long)k.N, (long long)k.K, k.epi, k.out, k.aligned, k.hilo, k.wpack, p.cand.name.c_str(), p.us);
    std::fclose(f);
}

std::vector<Candidate> candidates(const Key &k);
bool fits(const Candidate &c, const Key &k, size_t ws);

int load_plans(proj_ctx *c) {
    const char *path = std::getenv("PROJ_PLAN_FILE");
    if (!path || !*path) return 0;
    FILE *f = std::fopen(path, "r");
    if (!f) return 0;
    char line[512], dev[128], name[160];
    int loaded = 0;
    while (std::fgets(line, sizeof line, f)) {
        long long M, N, K;
        int ver, epi, out, al, hilo, wpack;
        float us;
        if (std::sscanf(line, "proj-plan %d %127s %lld %lld %lld %d %d %d %d %d %159s %f", &ver, dev, &M, &N, &K, &epi,
                        &out, &al, &hilo, &wpack, name, &us) != 12 ||
            ver != 1 || c->dev_id != dev || M <= 0 || N <= 0 || K < 0)
            continue;
        const Key k{M, N, K, epi, out, al, hilo, wpack};
        for (const Candidate &cand : candidates(k))
            if (cand.name == name && fits(cand, k, c->ws_bytes)) {
                c->plans[k] = Plan{cand, true, us};
                ++loaded;
                break;
            }
    }
    std::fclose(f);
    return loaded;
}

bool env_flag(const char *name, bool dflt) {
    const char *v = std::getenv(name);
    if (!v || !*v) return dflt;
    return !(v[0] == '0' || v[0] == 'n' || v[0] == 'N' || v[0] == 'f' || v[0] == 'F');
}

void set_err(proj_ctx *c, const char *fmt, ...) {
    if (!c) return;
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
}

proj_status hip_fail(proj_ctx *c, const char *what, hipError_t e) {
    set_err(c, "%s: %s", what, hipGetErrorString(e));
    return PROJ_ERR_HIP;
}

class DeviceGuard {
   public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
        if (prev_ != dev) hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) hipSetDevice(prev_);
    }

   private:
    int prev_ = -1;
};

// largest M offered to the streaming kernel (in 64- or 128-row blocks)
constexpr int64_t kStreamMaxM = 512;

int mt_for(int64_t M) {
    const int64_t need = (M + 15) / 16;
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 0;
}

std::string stream_name(const StreamVariant &v, int S, bool atomic = false, int walk = 0) {
    char b[96];
    snprintf(b, sizeof b, "stream_mt%d_nt%d_w%d_k%d_d%d%s_s%d%s", v.mt, v.nt, v.waves, v.kc, v.depth,
             v.wnt ? "_wnt" : "", S, atomic ? "_atomic" : "");
    std::string n = b;
    if (walk > 0) n += "_r" + std::to_string(walk);
    return n;
}

// K-walk strides offered for every streaming candidate: tile t starts at
// stage (stride x t) mod T.  Which one keeps the memory channels busiest
// depends on the shape and the W layout (stride 7 is best for the
// M16 N8192 decode shape, stride 1 for the M64 N28672 one, in a sweep of
// 1, 3, 5, 7, 11, 13, 17, 29 and a golden-ratio hash), so the measurement
// picks.  Stride 7 carries no suffix, stride 1 is suffixed _r1.
void push_stream(std::vector<Candidate> &out, int i, const StreamVariant &v, int S, int atomic) {
    for (int walk : {0, 1}) {
        Candidate c{KIND_STREAM, i, S, stream_name(v, S, atomic != 0, walk), atomic};
        c.walk = walk;
        out.push_back(c);
    }
}

// Split partials may be added into Y with fp32 atomics when Y is fp32 and
// the epilogue is additive (no GELU): the bias is then added by one split.
bool atomic_ok(const Key &k) { return k.out == PROJ_OUT_F32 && !(k.epi & 2); }

std::string gemv_name(const GemvVariant &v, int S) {
    char b[96];
    snprintf(b, sizeof b, "gemv_m%d_r%d_w%d_u%d%s_s%d", v.mr, v.rows, v.waves, v.unroll, v.wnt ? "_wnt" : "", S);
    return b;
}

std::string gemm_name(const GemmVariant &v, int S) {
    char b[96];
    snprintf(b, sizeof b, "%s_%dx%dx%d_w%dx%d_g%d", v.family, v.bm, v.bn, v.bk, v.waves_m, v.waves_n, v.group_m);
    std::string n = b;
    if (S > 1) n += "_s" + std::to_string(S);
    return n;
}

// Every compiled variant that can run this shape correctly.  These are
// validity rules only (operand alignment, tile coverage of M, 32-bit buffer
// offsets, a split covering at least one stage); the measurement picks among
// them.  Whether a split's fp32 partials fit a context's workspace is decided
// per context (workspace_bytes, fits).
std::vector<Candidate> candidates(const Key &k) {
    std::vector<Candidate> out;
    if (k.wpack) {
        // packed weights are read by the streaming kernel's buffer-resource
        // path only, with the tile height they were packed for
        const int mt = mt_for(k.M);
        if (!k.aligned || k.K <= 0 || k.K % 128 != 0 || (mt == 0 && k.M > kStreamMaxM)) return out;
        for (int i = 0; i < kNumStreamVariants; ++i) {
            const StreamVariant &v = kStreamVariants[i];
            if (v.nt != k.wpack || v.kc % 128 != 0 || k.K % v.kc != 0) continue;
            if (mt > 0 ? v.mt != mt : (v.mt != 4 && v.mt != 8)) continue;
            const int64_t rows_x = k.M < 16 * v.mt ? k.M : 16 * v.mt;
            if (rows_x * k.K * 2 >= (int64_t{1} << 32) || int64_t{16} * v.nt * k.K * 2 >= (int64_t{1} << 32)) continue;
            const int64_t mblocks = (k.M + 16 * v.mt - 1) / (16 * v.mt);
            const int64_t stages = k.K / v.kc;
            const int64_t tiles = (k.N + 16 * v.nt - 1) / (16 * v.nt);
            for (int S : {1, 2, 4, 8, 16}) {
                if (S > 1 && S > stages) continue;
                if (mblocks * tiles * S > 0x7fffffff) continue;
                push_stream(out, i, v, S, 0);
                if (S > 1 && atomic_ok(k)) push_stream(out, i, v, S, 1);
            }
        }
        return out;
    }
    if (k.aligned && k.K > 0) {
        // row blocks of the streaming kernel: the one block size that covers
        // M up to 64 rows; above that, 64- or 128-row blocks up to
        // kStreamMaxM rows (one block of W rows is then read once per row
        // block)
        const int mt = mt_for(k.M);
        auto mt_ok = [&](int vmt) { return mt > 0 ? vmt == mt : k.M <= kStreamMaxM && (vmt == 4 || vmt == 8); };
        if (mt > 0 || k.M <= kStreamMaxM) {
            for (int i = 0; i < kNumStreamVariants; ++i) {
                const StreamVariant &v = kStreamVariants[i];
                if (!mt_ok(v.mt)) continue;
                const int64_t mblocks = (k.M + 16 * v.mt - 1) / (16 * v.mt);
                const int64_t rows_x = k.M < 16 * v.mt ? k.M : 16 * v.mt;
                // a hi/lo pair is read on the buffer-resource path only: whole
                // stages, the X wrap at K/2 on a stage boundary, and operand
                // offsets that fit its 32-bit resources
                if (k.hilo && (k.K % v.kc != 0 || (k.K / 2) % v.kc != 0 ||
                               rows_x * (k.K / 2) * 2 >= (int64_t{1} << 32) ||
                               int64_t{16} * v.nt * k.K * 2 >= (int64_t{1} << 32)))
                    continue;
                const int64_t stages = (k.K + v.kc - 1) / v.kc;
                const int64_t tiles = (k.N + 16 * v.nt - 1) / (16 * v.nt);
                for (int S : {1, 2, 4, 8, 16}) {
                    if (S > 1 && S > stages) continue;
                    if (mblocks * tiles * S > 0x7fffffff) continue;
                    push_stream(out, i, v, S, 0);
                    if (S > 1 && atomic_ok(k)) push_stream(out, i, v, S, 1);
                }
            }
        }
        // register-streaming GEMV: the smallest token-row count that covers
        // M (up to 8), whole 16-byte chunks, offsets in the 31-bit range
        const int mr = k.M <= 1 ? 1 : k.M <= 2 ? 2 : k.M <= 4 ? 4 : k.M <= 8 ? 8 : 0;
        const int64_t kxk = k.hilo ? k.K / 2 : k.K;
        if (mr > 0 && kxk % 8 == 0 && k.M * kxk * 2 <= 0x7fffffff) {
            for (int i = 0; i < kNumGemvVariants; ++i) {
                const GemvVariant &v = kGemvVariants[i];
                if (v.mr != mr || static_cast<int64_t>(v.rows) * k.K * 2 > 0x7fffffff) continue;
                const int64_t tiles = (k.N + v.rows - 1) / v.rows;
                for (int S : {1, 2, 4, 8}) {
                    if (S > 1 && S > k.K / 8) continue;
                    if (tiles * S > 0x7fffffff) continue;
                    out.push_back({KIND_GEMV, i, S, gemv_name(v, S)});
                }
            }
        }
        for (int i = 0; i < kNumGemmVariants; ++i) {
            const GemmVariant &v = kGemmVariants[i];
            if (k.K % v.kmult != 0) continue;
            // the persistent kernels (families gemmpp64p and gemmpp64d) are the
            // GEMMs that read a hi/lo pair
            const bool persistent = std::strncmp(v.family, "gemmpp64", 8) == 0 && v.family[8] != '\0';
            if (k.hilo && (!persistent || (k.K / 2) % 64 != 0 || k.K < 128)) continue;
            if (v.kmax > 0 && k.K > v.kmax) continue;
            out.push_back({KIND_GEMM, i, 1, gemm_name(v, 1)});
            // K splits: at least two 64-wide k-ranges each
            const int64_t tiles = ((k.M + v.bm - 1) / v.bm) * ((k.N + v.bn - 1) / v.bn);
            for (int S = 2; S <= v.max_splits; S *= 2) {
                if (k.K / 64 < 2 * static_cast<int64_t>(S)) break;
                if (tiles * S > 0x7fffffff) break;
                out.push_back({KIND_GEMM, i, S, gemm_name(v, S)});
            }
        }
    }
    if (out.empty()) out.push_back({KIND_GENERIC, 0, 1, "generic"});
    return out;
}

// Bytes of fp32 partials a candidate writes to the split-K workspace.
size_t workspace_bytes(const Candidate &c, const Key &k) {
    if (c.splits <= 1 || c.atomic) return 0;
    return static_cast<size_t>(c.splits) * static_cast<size_t>(k.M) * static_cast<size_t>(k.N) * sizeof(float);
}

// Whether a candidate can run with `ws` bytes of split-K workspace.
bool fits(const Candidate &c, const Key &k, size_t ws) { return workspace_bytes(c, k) <= ws; }

// The candidates that can run with `ws` bytes of split-K workspace (the
// any-shape kernel, which needs none, when nothing else does).
std::vector<Candidate> candidates_within(const Key &k, size_t ws) {
    std::vector<Candidate> all = candidates(k), out;
    for (const Candidate &c : all)
        if (fits(c, k, ws)) out.push_back(c);
    if (out.empty()) out.push_back({KIND_GENERIC, 0, 1, "generic"});
    return out;
}

// The untimed plan used under stream capture or with PROJ_TUNE=0, among the
// candidates that fit `ws` bytes of workspace on a device of `cus` compute
// units.
Candidate default_candidate(const Key &k, size_t ws, int cus) {
    std::vector<Candidate> c = candidates_within(k, ws);
    auto find = [&](const char *name) -> const Candidate * {
        for (const Candidate &x : c)
            if (x.name == name) return &x;
        return nullptr;
    };
    if (mt_for(k.M) > 0) {
        // 32 rows per workgroup, 256-byte row segments, non-temporal W if
        // such a variant exists for this M (else 5 stages in flight), and
        // the smallest split count that gives every CU a workgroup
        for (int pass = 0; pass < 2; ++pass)
            for (const Candidate &x : c) {
                if (x.kind != KIND_STREAM) continue;
                const StreamVariant &v = kStreamVariants[x.variant];
                if (v.nt != 2 || v.kc != 128 || v.waves != 4) continue;
                if (pass == 0 ? !v.wnt : (v.wnt || v.depth != 5)) continue;
                if (((k.N + 31) / 32) * x.splits >= cus || x.splits == 8) return x;
            }
    }
    if (const Candidate *g = find("gemmpp64_256x256x64_w4x2_g4")) return *g;
    if (const Candidate *g = find("gemmpp_256x256x32_w4x2_g4")) return *g;
    if (const Candidate *g = find("gemm_256x256x64_w2x2_g4")) return *g;
    for (const Candidate &x : c)
        if (x.kind == KIND_GEMM) return x;
    return c.front();
}

proj_status no_workspace(proj_ctx *c, const Candidate &cand, const Key &k) {
    set_err(c, "%s needs %zu bytes of split-K workspace; the context holds %zu (proj_create's bound)",
            cand.name.c_str(), workspace_bytes(cand, k), c->ws_bytes);
    return PROJ_ERR_NO_MEMORY;
}

Args make_args(proj_ctx *c, const void *X, const void *W, const void *bias, int epi, int64_t M, int64_t N,
               int64_t K, void *Y, int out, int hilo = 0, int wpack = 0) {
    Args a;
    a.kx = hilo ? K / 2 : K;
    a.wpack = static_cast<int16_t>(wpack);
    a.X = static_cast<const uint16_t *>(X);
    a.W = static_cast<const uint16_t *>(W);
    a.bias = static_cast<const uint16_t *>(bias);
    a.Y = Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.epi = epi;
    a.out = out;
    a.ws = c->ws;
    a.zeros = c->zeros;
    return a;
}

hipError_t launch(const Candidate &cand, const Args &a, hipStream_t st) {
    switch (cand.kind) {
        case KIND_GEMM: return kGemmVariants[cand.variant].launch(a, cand.splits, st);
        case KIND_STREAM: {
            Args b = a;
            b.atomic = cand.atomic;
            b.walk = static_cast<int16_t>(cand.walk);
            return kStreamVariants[cand.variant].launch(b, cand.splits, st);
        }
        case KIND_GEMV: return kGemvVariants[cand.variant].launch(a, cand.splits, st);
        default: return launch_generic(a, st);
    }
}

// Whether byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// K is the product depth (twice the X row length for a hi/lo pair); wpack
// the packed weights' tile height (0: row-major W).
proj_status check_args(proj_ctx *c, const void *X, const void *W, const void *bias, int epi, int64_t M,
                       int64_t N, int64_t K, void *Y, int out, int hilo = 0, int wpack = 0) {
    if (!c) return PROJ_ERR_INVALID_ARG;
    if (c->magic == kDead) return PROJ_ERR_DESTROYED;
    if (c->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) {
        set_err(c, "negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
        return PROJ_ERR_INVALID_ARG;
    }
    if (epi < PROJ_EPI_NONE || epi > PROJ_EPI_BIAS_GELU_TANH) {
        set_err(c, "unknown epilogue %d", epi);
        return PROJ_ERR_INVALID_ARG;
    }
    if (out != PROJ_OUT_F32 && out != PROJ_OUT_BF16) {
        set_err(c, "unknown output dtype %d", out);
        return PROJ_ERR_INVALID_ARG;
    }
    if (M == 0 || N == 0) return PROJ_OK;
    if (!Y) {
        set_err(c, "Y is NULL");
        return PROJ_ERR_INVALID_ARG;
    }
    if (K > 0 && (!X || !W)) {
        set_err(c, "X or W is NULL");
        return PROJ_ERR_INVALID_ARG;
    }
    if ((epi & 1) && !bias) {
        set_err(c, "epilogue %d needs a bias, got NULL", epi);
        return PROJ_ERR_INVALID_ARG;
    }
    const uintptr_t yal = out == PROJ_OUT_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(Y) % yal || reinterpret_cast<uintptr_t>(X) % 2 ||
        reinterpret_cast<uintptr_t>(W) % 2 || reinterpret_cast<uintptr_t>(bias) % 2) {
        set_err(c, "a pointer is not aligned to its element size");
        return PROJ_ERR_INVALID_ARG;
    }
    if (M > (int64_t(1) << 40) / (N > 0 ? N : 1)) {
        set_err(c, "M*N too large");
        return PROJ_ERR_UNSUPPORTED;
    }
    // Y is written (several times while a plan is measured), so it must not
    // share memory with an input
    if (K <= (int64_t(1) << 40) / (M > N ? M : N)) {
        const uint64_t ybytes = static_cast<uint64_t>(M) * N * (out == PROJ_OUT_F32 ? 4 : 2);
        const uint64_t xbytes = static_cast<uint64_t>(M) * (hilo ? K / 2 : K) * 2;
        const int64_t pb = wpack ? proj_packed_bytes(N, K, wpack) : -1;
        const uint64_t wbytes = pb >= 0 ? static_cast<uint64_t>(pb) : static_cast<uint64_t>(N) * K * 2;
        const uint64_t bbytes = (epi & 1) ? static_cast<uint64_t>(N) * 2 : 0;
        if (overlap(Y, ybytes, X, xbytes) || overlap(Y, ybytes, W, wbytes) || overlap(Y, ybytes, bias, bbytes)) {
            set_err(c, "Y overlaps X, W or bias");
            return PROJ_ERR_INVALID_ARG;
        }
    }
    return PROJ_OK;
}

Key make_key(const void *X, const void *W, int epi, int64_t M, int64_t N, int64_t K, int out, int hilo = 0,
             int wpack = 0) {
    const bool al = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && (reinterpret_cast<uintptr_t>(W) % 16 == 0) &&
                    ((hilo ? K / 2 : K) % 8 == 0);
    return Key{M, N, K, epi, out, al ? 1 : 0, hilo, wpack};
}

bool capturing(hipStream_t st) {
    hipStreamCaptureStatus s = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &s) != hipSuccess) return false;
    return s != hipStreamCaptureStatusNone;
}

// Workgroups of a candidate's main kernel, and the M x N extent its matrix
// operations actually cover (whole tiles, padded past M and N).
struct Extent {
    int64_t wgs, mp, np;
};
Extent candidate_extent(const Candidate &c, const Key &k) {
    auto up = [](int64_t x, int64_t t) { return (x + t - 1) / t * t; };
    switch (c.kind) {
        case KIND_STREAM: {
            const StreamVariant &v = kStreamVariants[c.variant];
            const int64_t mp = up(k.M, 16 * v.mt), np = up(k.N, 16 * v.nt);
            return {mp / (16 * v.mt) * (np / (16 * v.nt)) * c.splits, mp, np};
        }
        case KIND_GEMV: {
            const GemvVariant &v = kGemvVariants[c.variant];
            const int64_t np = up(k.N, v.rows);
            return {np / v.rows * c.splits, static_cast<int64_t>(v.mr), np};
        }
        case KIND_GEMM: {
            const GemmVariant &v = kGemmVariants[c.variant];
            const int64_t mp = up(k.M, v.bm), np = up(k.N, v.bn);
            return {mp / v.bm * (np / v.bn) * c.splits, mp, np};
        }
        default:
            return {(k.M * k.N + 255) / 256, k.M, k.N};
    }
}

// A time no run of the candidate can beat: the multiply-adds its tiles
// cover (2 Mp Np K) at one CU's dense bf16 matrix rate (cu_flops, from the
// device clock) on each CU it occupies.  The tuner does not launch
// candidates whose bound is far above the best time already measured (a
// 256-row GEMM tile walking a very long K for 16 token rows alone would take
// milliseconds to seconds).
double lower_bound_us(const Candidate &c, const Key &k, int cus, double cu_flops) {
    const Extent e = candidate_extent(c, k);
    const double wgs = std::max<double>(1.0, std::min<double>(static_cast<double>(e.wgs), cus));
    return 2.0 * static_cast<double>(e.mp) * static_cast<double>(e.np) * static_cast<double>(k.K) /
           (wgs * cu_flops) * 1e6;
}
constexpr double kSkipFactor = 20.0;

// Time every candidate that fits the context's workspace on the caller's
// buffers; returns the winner.  The last-level cache is flushed before each
// timed run when the operands could fit in it, so small shapes are timed as
// they run from HBM: the flush buffer (kFlushBytes) is allocated for the
// tuning run, and exchanged for the operand copies of the graph timing
// (below, together no more than kFlushBytes), all freed before returning.
proj_status tune(proj_ctx *c, const Key &k, const Args &a, hipStream_t st, Plan &plan) {
    std::vector<Candidate> cands = candidates_within(k, c->ws_bytes);
    const size_t bytes = static_cast<size_t>(2 * (k.M + k.N) * k.K);
    void *fbuf = nullptr;
    if (bytes < kFlushBytes && hipMalloc(&fbuf, kFlushBytes + 1024) != hipSuccess) {
        (void)hipGetLastError();
        fbuf = nullptr;  // tune without flushing
    }
    struct FreeAfter {
        void *p;
        ~FreeAfter() {
            if (p) hipFree(p);
        }
    } free_after{fbuf};
    unsigned *sink = fbuf ? reinterpret_cast<unsigned *>(static_cast<char *>(fbuf) + kFlushBytes) : nullptr;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return hip_fail(c, "hipEventCreate", hipGetLastError());
    if (hipEventCreate(&e1) != hipSuccess) {
        hipEventDestroy(e0);
        return hip_fail(c, "hipEventCreate", hipGetLastError());
    }
    // one timed run of candidate i (after a cache flush where that applies);
    // a negative time if it could not run
    auto time_once = [&](size_t i) -> float {
        if (fbuf) launch_flush(fbuf, kFlushBytes, sink, st);
        hipEventRecord(e0, st);
        if (launch(cands[i], a, st) != hipSuccess) return -1.f;
        hipEventRecord(e1, st);
        float ms = 0.f;
        if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1.f;
        return ms * 1000.f;
    };
    auto median = [](std::vector<float> &t) {
        std::sort(t.begin(), t.end());
        return t[t.size() / 2];
    };
    // pass 1: every candidate, a few runs each (except those whose lower
    // bound is already far behind the best median so far)
    std::vector<std::pair<float, size_t>> ranked;
    float best_so_far = -1.f;
    for (size_t i = 0; i < cands.size(); ++i) {
        if (best_so_far > 0.f && lower_bound_us(cands[i], k, c->cus, c->cu_flops) > kSkipFactor * best_so_far)
            continue;
        if (launch(cands[i], a, st) != hipSuccess) {  // warm-up; skip variants that cannot launch
            (void)hipGetLastError();
            continue;
        }
        std::vector<float> t;
        for (int r = 0; r < 7; ++r) {
            const float us = time_once(i);
            if (us < 0.f) break;
            t.push_back(us);
        }
        if (t.size() < 7) {
            (void)hipGetLastError();
            continue;
        }
        ranked.push_back({median(t), i});
        if (best_so_far < 0.f || ranked.back().first < best_so_far) best_so_far = ranked.back().first;
    }
    if (ranked.empty()) {
        hipEventDestroy(e0);
        hipEventDestroy(e1);
        set_err(c, "no candidate could be launched");
        return PROJ_ERR_HIP;
    }
    // pass 2: the leaders again, interleaved round by round so that clock
    // and thermal drift over the tuning run falls on all of them alike.
    // Where P >= 2 sets of the operands fill at least half of kFlushBytes
    // (more than the last-level cache), each leader is timed as a model
    // replays it: a HIP graph of calls cycling over the caller's operands
    // and P - 1 copies, so
    // every call reads its operands from HBM and back-to-back kernels
    // (split-K passes, zero fills) run with graph launch gaps.  The graph
    // holds about 400 us of calls (a whole number of cycles, at most 256
    // calls), so the launch and event overhead of one measurement, which
    // varies by a few microseconds, is spread over many calls: with one
    // cycle of 3 calls it reordered plans 7% apart.  Single cold launches
    // carry a launch overhead of their own that reorders plans of a few
    // microseconds.  Otherwise the leaders are timed as in pass 1.
    std::sort(ranked.begin(), ranked.end());
    // Set 0 of the graph is the caller's buffers; the other sets are copies,
    // each operand in an allocation of its own.  Where W sits in memory
    // changes which ring depth wins: with the copies carved out of one
    // 512 MiB allocation on 2 MiB boundaries, the M=16 K=8192 N=8192 decode
    // plans came out within 1% of each other (22.8-23.8 us), while with
    // allocations of their own, as a framework's tensors have, the 4-stage
    // ring led the 256-column 8-wave form by 7% (21.8 against 23.3 us), as in
    // use.
    auto up2m = [](size_t x) { return (x + (size_t{2} << 20) - 1) / (size_t{2} << 20) * (size_t{2} << 20); };
    const size_t xb = static_cast<size_t>(a.M) * static_cast<size_t>(a.kx) * 2;
    const size_t wb = a.wpack ? static_cast<size_t>(proj_packed_bytes(a.N, a.K, a.wpack))
                              : static_cast<size_t>(a.N) * static_cast<size_t>(a.K) * 2;
    const size_t bb = (a.epi & 1) ? static_cast<size_t>(a.N) * 2 : 0;
    const size_t set = up2m(xb) + up2m(wb) + up2m(bb);
    const size_t P = (fbuf && st && set > 0) ? std::min<size_t>(256, kFlushBytes / set) : 0;
    const bool graphs = P >= 2 && P * set >= kFlushBytes / 2;
    // 16 leaders where graph timing applies: cold single launches rank some
    // plan families (workspace splits against atomic splits, the two K-walk
    // starts of a streaming variant) differently from graph replay, so the
    // pass-1 top must be wide enough to hold each family's best
    const size_t lead = std::min(ranked.size(), graphs ? size_t{16} : size_t{4});
    std::vector<std::vector<float>> t2(lead);
    bool graphed = false;
    size_t cycles = 1;
    if (graphs) {
        const double per_cycle_us = std::max(1.0, static_cast<double>(ranked[0].first) * static_cast<double>(P));
        cycles = std::max<size_t>(1, std::min<size_t>(256 / P, static_cast<size_t>(std::ceil(400.0 / per_cycle_us))));
    }
    const size_t L = P * cycles;  // calls per graph
    // copies for the graph sets, freed when tuning returns
    struct FreeAll {
        std::vector<void *> p;
        ~FreeAll() {
            for (void *q : p) hipFree(q);
        }
    } copies;
    if (graphs) {
        // the flush buffer is not read from here on (a fallback to single
        // launches then runs without the flush): let it go before the copies
        // are allocated, so tuning holds at most 512 MiB of either
        if (hipStreamSynchronize(st) == hipSuccess) {
            hipFree(fbuf);
            free_after.p = fbuf = nullptr;
            sink = nullptr;
        }
        std::vector<Args> sets(P, a);
        bool ok = true;
        auto alloc = [&](size_t n) -> char * {
            void *q = nullptr;
            if (n == 0) return nullptr;
            if (hipMalloc(&q, n) != hipSuccess) {
                (void)hipGetLastError();
                return nullptr;
            }
            copies.p.push_back(q);
            return static_cast<char *>(q);
        };
        for (size_t p = 1; p < P && ok; ++p) {
            char *x = alloc(xb), *w = alloc(wb), *b = alloc(bb);
            ok = x && w && (bb == 0 || b) &&
                 hipMemcpyAsync(x, a.X, xb, hipMemcpyDeviceToDevice, st) == hipSuccess &&
                 hipMemcpyAsync(w, a.W, wb, hipMemcpyDeviceToDevice, st) == hipSuccess &&
                 (bb == 0 || hipMemcpyAsync(b, a.bias, bb, hipMemcpyDeviceToDevice, st) == hipSuccess);
            sets[p].X = reinterpret_cast<const uint16_t *>(x);
            sets[p].W = reinterpret_cast<const uint16_t *>(w);
            if (bb) sets[p].bias = reinterpret_cast<const uint16_t *>(b);
        }
        std::vector<hipGraphExec_t> ex(lead, nullptr);
        for (size_t j = 0; j < lead && ok; ++j) {
            if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) {
                ok = false;
                break;
            }
            bool launched = true;
            for (size_t q = 0; q < L && launched; ++q) launched = launch(cands[ranked[j].second], sets[q % P], st) == hipSuccess;
            hipGraph_t gr = nullptr;
            const bool ended = hipStreamEndCapture(st, &gr) == hipSuccess;
            ok = launched && ended && gr && hipGraphInstantiate(&ex[j], gr, nullptr, nullptr, 0) == hipSuccess;
            if (gr) hipGraphDestroy(gr);
        }
        for (size_t j = 0; j < lead && ok; ++j) ok = hipGraphLaunch(ex[j], st) == hipSuccess;  // first replay
        ok = ok && hipStreamSynchronize(st) == hipSuccess;
        for (int r = 0; r < 15 && ok; ++r)
            for (size_t j = 0; j < lead && ok; ++j) {
                float ms = 0.f;
                ok = hipEventRecord(e0, st) == hipSuccess && hipGraphLaunch(ex[j], st) == hipSuccess &&
                     hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
                     hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
                if (ok) t2[j].push_back(ms * 1000.f / static_cast<float>(L));
            }
        for (hipGraphExec_t x : ex)
            if (x) hipGraphExecDestroy(x);
        (void)hipGetLastError();
        graphed = ok;
        if (!ok) {
            hipStreamSynchronize(st);
            for (auto &t : t2) t.clear();
        }
    }
    if (!graphed)
        for (int r = 0; r < 15; ++r)
            for (size_t j = 0; j < lead; ++j) {
                const float us = time_once(ranked[j].second);
                if (us >= 0.f) t2[j].push_back(us);
            }
    (void)hipGetLastError();
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    float best = ranked[0].first;
    size_t best_i = ranked[0].second;
    bool first = true;
    for (size_t j = 0; j < lead; ++j) {
        if (t2[j].empty()) continue;
        const float med = median(t2[j]);
        if (first || med < best) {
            best = med;
            best_i = ranked[j].second;
            first = false;
        }
    }
    plan = Plan{cands[best_i], true, best};
    // leave the winner's result in Y (and let the flush buffer go only once
    // the timed runs that read it are done)
    hipError_t e = launch(plan.cand, a, st);
    if (e != hipSuccess) return hip_fail(c, "launch", e);
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(c, "hipStreamSynchronize", e);
    return PROJ_OK;
}

proj_status run_impl(proj_ctx *c, const void *X, const void *W, const void *bias, int epi, int64_t M, int64_t N,
                     int64_t K, void *Y, int out, void *stream, bool force_tune, int hilo = 0, int wpack = 0) {
    proj_status s = check_args(c, X, W, bias, epi, M, N, K, Y, out, hilo, wpack);
    if (s != PROJ_OK || M == 0 || N == 0) return s;
    DeviceGuard g(c->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Key k = make_key(X, W, epi, M, N, K, out, hilo, wpack);
    const Args a = make_args(c, X, W, bias, epi, M, N, K, Y, out, hilo, wpack);
    if (wpack && candidates(k).empty()) {
        set_err(c, "no kernel reads packed weights for M=%lld K=%lld (M <= %lld, K a multiple of 128, "
                   "16-byte aligned X and W)", (long long)M, (long long)K, (long long)kStreamMaxM);
        return PROJ_ERR_UNSUPPORTED;
    }
    const bool cap = capturing(st);
    if (force_tune && cap) {
        set_err(c, "cannot tune while the stream is capturing");
        return PROJ_ERR_NOT_TUNED;
    }
    std::lock_guard<std::mutex> lock(c->mu);
    auto it = c->plans.find(k);
    if (it == c->plans.end() || (force_tune && !it->second.tuned)) {
        Plan p;
        if (!cap && (force_tune || env_flag("PROJ_TUNE", true))) {
            s = tune(c, k, a, st, p);
            if (s != PROJ_OK) return s;
            c->plans[k] = p;
            save_plan(c, k, p);
            if (plan_log())
                std::fprintf(stderr, "proj: M=%lld N=%lld K=%lld epi=%d out=%d hilo=%d wpack=%d: tuned %s %.2f us\n",
                             (long long)M, (long long)N, (long long)K, epi, out, hilo, wpack, p.cand.name.c_str(), p.us);
            return PROJ_OK;  // tune() already left the winner's result in Y
        }
        p = Plan{default_candidate(k, c->ws_bytes, c->cus), false, 0.f};
        it = c->plans.insert_or_assign(k, p).first;
        if (plan_log())
            std::fprintf(stderr, "proj: M=%lld N=%lld K=%lld epi=%d out=%d hilo=%d wpack=%d: default %s (%s)\n",
                         (long long)M, (long long)N, (long long)K, epi, out, hilo, wpack, p.cand.name.c_str(),
                         cap ? "stream capture" : "PROJ_TUNE=0");
    } else if (force_tune) {
        // already tuned: just run it
    }
    hipError_t e = launch(it->second.cand, a, st);
    if (e != hipSuccess) return hip_fail(c, "launch", e);
    return PROJ_OK;
}

// ---- allocation-free runs: the device address of `scratch` on each device
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device` (which must be current); resolved
// on the first call per device.
hipError_t scratch_address(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

extern "C" {

proj_status proj_create(proj_ctx **out, int device, size_t max_workspace_bytes) {
    if (!out) return PROJ_ERR_INVALID_ARG;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return PROJ_ERR_HIP;
    if (device < 0 || device >= n) return PROJ_ERR_INVALID_ARG;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return PROJ_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PROJ_ERR_UNSUPPORTED;
    DeviceGuard g(device);
    proj_ctx *c = new (std::nothrow) proj_ctx();
    if (!c) return PROJ_ERR_NO_MEMORY;
    c->magic = kMagic;
    c->device = device;
    c->cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    // each CU's 4 SIMDs issue one 16x16x32 bf16 matrix op (16,384 flops)
    // every 16 cycles; clockRate is in kHz
    c->cu_flops = 4.0 * 16384.0 / 16.0 * (prop.clockRate > 0 ? prop.clockRate : 1) * 1e3;
    c->ws = nullptr;
    c->ws_bytes = 0;
    c->zeros = nullptr;
    c->scratch_dev = nullptr;
    if (scratch_address(device, &c->scratch_dev) != hipSuccess) {
        (void)hipGetLastError();
        delete c;
        return PROJ_ERR_HIP;
    }
    bool ok = hipMalloc(&c->zeros, kZeroBytes + kSinkBytes) == hipSuccess &&
              hipMemset(c->zeros, 0, kZeroBytes + kSinkBytes) == hipSuccess;
    if (ok && max_workspace_bytes > 0) {
        const size_t ws = max_workspace_bytes / 256 * 256;
        if (ws > 0 && hipMalloc(&c->ws, ws) != hipSuccess) {
            (void)hipGetLastError();
            hipFree(c->zeros);
            delete c;
            return PROJ_ERR_NO_MEMORY;
        }
        c->ws_bytes = ws;
    }
    for (int i = 0; ok && i < kNumGemmVariants; ++i) ok = kGemmVariants[i].prepare() == hipSuccess;
    for (int i = 0; ok && i < kNumStreamVariants; ++i) ok = kStreamVariants[i].prepare() == hipSuccess;
    ok = ok && hipDeviceSynchronize() == hipSuccess;
    if (!ok) {
        hipFree(c->ws);
        hipFree(c->zeros);
        delete c;
        return PROJ_ERR_HIP;
    }
    c->dev_id = std::string(prop.gcnArchName) + "_cu" + std::to_string(c->cus);
    for (char &ch : c->dev_id)
        if (ch == ' ') ch = '_';
    const int loaded = load_plans(c);
    if (plan_log() && loaded)
        std::fprintf(stderr, "proj: %d plans for %s loaded from %s\n", loaded, c->dev_id.c_str(),
                     std::getenv("PROJ_PLAN_FILE"));
    *out = c;
    return PROJ_OK;
}

proj_status proj_run(proj_ctx *ctx, const void *X, const void *W, const void *bias, int epilogue, int64_t M,
                     int64_t N, int64_t K, void *Y, int out_dtype, void *stream) {
    return run_impl(ctx, X, W, bias, epilogue, M, N, K, Y, out_dtype, stream, false);
}

proj_status proj_run_noalloc(proj_ctx *ctx, const void *X, const void *W, const void *bias, int epilogue,
                             int64_t M, int64_t N, int64_t K, void *Y, int out_dtype, void *stream) {
    proj_status s = check_args(ctx, X, W, bias, epilogue, M, N, K, Y, out_dtype);
    if (s != PROJ_OK || M == 0 || N == 0) return s;
    DeviceGuard g(ctx->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Key k = make_key(X, W, epilogue, M, N, K, out_dtype);
    Candidate cand;
    {
        std::lock_guard<std::mutex> lock(ctx->mu);
        auto it = ctx->plans.find(k);
        // the plan proj_run runs for this shape, or (none cached yet) the
        // default plan among those whose partials fit the scratch, not cached
        cand = it != ctx->plans.end()
                   ? it->second.cand
                   : default_candidate(k, std::min(ctx->ws_bytes, kScratchBytes), ctx->cus);
    }
    if (workspace_bytes(cand, k) > kScratchBytes) {
        set_err(ctx, "%s writes %zu bytes of split-K partials; proj_run_noalloc's static scratch holds %zu",
                cand.name.c_str(), workspace_bytes(cand, k), kScratchBytes);
        return PROJ_ERR_NO_MEMORY;
    }
    Args a = make_args(ctx, X, W, bias, epilogue, M, N, K, Y, out_dtype);
    a.ws = static_cast<float *>(ctx->scratch_dev);
    hipError_t e = launch(cand, a, st);
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_tune(proj_ctx *ctx, const void *X, const void *W, const void *bias, int epilogue, int64_t M,
                      int64_t N, int64_t K, void *Y, int out_dtype, void *stream) {
    return run_impl(ctx, X, W, bias, epilogue, M, N, K, Y, out_dtype, stream, true);
}

proj_status proj_prepare_hilo(proj_ctx *ctx, const float *W, int64_t N, int64_t K, void *Whl, void *stream) {
    if (!ctx) return PROJ_ERR_INVALID_ARG;
    if (ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (ctx->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    if (N < 0 || K < 0) {
        set_err(ctx, "negative size N=%lld K=%lld", (long long)N, (long long)K);
        return PROJ_ERR_INVALID_ARG;
    }
    if (N == 0 || K == 0) return PROJ_OK;
    if (!W || !Whl || reinterpret_cast<uintptr_t>(W) % 4 || reinterpret_cast<uintptr_t>(Whl) % 2) {
        set_err(ctx, "W or Whl is NULL or not aligned to its element size");
        return PROJ_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    hipError_t e = launch_hilo_split(W, N, K, static_cast<uint16_t *>(Whl), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_run_hilo(proj_ctx *ctx, const void *X, const void *Whl, const void *bias, int epilogue, int64_t M,
                          int64_t N, int64_t K, void *Y, int out_dtype, void *stream) {
    if (K < 0 || K > (int64_t(1) << 40)) return PROJ_ERR_INVALID_ARG;
    return run_impl(ctx, X, Whl, bias, epilogue, M, N, 2 * K, Y, out_dtype, stream, false, 1);
}

// Tile heights (in 16-row units) that some streaming variant reads.
static bool packable_tile(int t) {
    for (int i = 0; i < kNumStreamVariants; ++i)
        if (kStreamVariants[i].nt == t && kStreamVariants[i].kc % 128 == 0) return true;
    return false;
}

int64_t proj_packed_bytes(int64_t N, int64_t K, int tile16) {
    if (N < 0 || K < 0 || K % 128 != 0 || !packable_tile(tile16) || N > (int64_t(1) << 40) / (K > 0 ? K : 1))
        return -1;
    const int64_t R = 16 * static_cast<int64_t>(tile16);
    return ((N + R - 1) / R) * R * K * 2;
}

proj_status proj_pack_weights(proj_ctx *ctx, const void *W, int64_t N, int64_t K, int tile16, void *Wp,
                              void *stream) {
    if (!ctx) return PROJ_ERR_INVALID_ARG;
    if (ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (ctx->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    if (proj_packed_bytes(N, K, tile16) < 0) {
        set_err(ctx, "cannot pack N=%lld K=%lld in tiles of %d x 16 rows (K must be a multiple of 128; "
                     "tile heights: those of the streaming kernel)", (long long)N, (long long)K, tile16);
        return PROJ_ERR_INVALID_ARG;
    }
    if (N == 0 || K == 0) return PROJ_OK;
    if (!W || !Wp || reinterpret_cast<uintptr_t>(W) % 16 || reinterpret_cast<uintptr_t>(Wp) % 16) {
        set_err(ctx, "W or Wp is NULL or not 16-byte aligned");
        return PROJ_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    hipError_t e = launch_pack(static_cast<const uint16_t *>(W), N, K, 16 * tile16, static_cast<uint16_t *>(Wp),
                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_run_packed(proj_ctx *ctx, const void *X, const void *Wp, int tile16, const void *bias, int epilogue,
                            int64_t M, int64_t N, int64_t K, void *Y, int out_dtype, void *stream) {
    if (!packable_tile(tile16)) {
        if (ctx && ctx->magic == kMagic) set_err(ctx, "no streaming variant reads tiles of %d x 16 rows", tile16);
        return PROJ_ERR_INVALID_ARG;
    }
    return run_impl(ctx, X, Wp, bias, epilogue, M, N, K, Y, out_dtype, stream, false, 0, tile16);
}

proj_status proj_destroy(proj_ctx *ctx) {
    if (!ctx) return PROJ_ERR_INVALID_ARG;
    if (ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (ctx->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    {
        DeviceGuard g(ctx->device);
        hipDeviceSynchronize();
        hipFree(ctx->ws);
        hipFree(ctx->zeros);
    }
    // the struct itself stays allocated as a marker, so a later use or a
    // second destroy of this handle (or a replay of one of its graphs) reads
    // valid memory and is reported
    std::lock_guard<std::mutex> lock(ctx->mu);
    ctx->ws = nullptr;
    ctx->ws_bytes = 0;
    ctx->zeros = nullptr;
    std::map<Key, Plan>().swap(ctx->plans);
    ctx->magic = kDead;
    return PROJ_OK;
}

const char *proj_status_string(int s) {
    switch (s) {
        case PROJ_OK: return "ok";
        case PROJ_ERR_INVALID_ARG: return "invalid argument";
        case PROJ_ERR_UNSUPPORTED: return "unsupported";
        case PROJ_ERR_HIP: return "HIP runtime error";
        case PROJ_ERR_NO_MEMORY: return "out of memory or workspace";
        case PROJ_ERR_NOT_TUNED: return "cannot tune while capturing";
        case PROJ_ERR_DESTROYED: return "handle already destroyed";
        default: return "unknown status";
    }
}

const char *proj_last_error(const proj_ctx *ctx) {
    if (!ctx || ctx->magic != kMagic) return "";
    return ctx->err.c_str();
}

static proj_status get_plan(proj_ctx *ctx, const Key &key, char *buf, size_t len) {
    if (ctx && ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (!ctx || ctx->magic != kMagic || !buf || len == 0) return PROJ_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(ctx->mu);
    auto it = ctx->plans.find(key);
    if (it == ctx->plans.end()) return PROJ_ERR_INVALID_ARG;
    char tmp[256];
    if (it->second.tuned)
        snprintf(tmp, sizeof tmp, "%s (tuned %.2fus)", it->second.cand.name.c_str(), it->second.us);
    else
        snprintf(tmp, sizeof tmp, "%s (default)", it->second.cand.name.c_str());
    if (std::strlen(tmp) + 1 > len) return PROJ_ERR_INVALID_ARG;
    std::strcpy(buf, tmp);
    return PROJ_OK;
}

proj_status proj_get_plan(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16,
                          char *buf, size_t len) {
    return get_plan(ctx, Key{M, N, K, epi, out, aligned16 ? 1 : 0}, buf, len);
}

proj_status proj_get_plan_hilo(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16,
                               char *buf, size_t len) {
    return get_plan(ctx, Key{M, N, 2 * K, epi, out, aligned16 ? 1 : 0, 1}, buf, len);
}

int proj_num_candidates(int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16) {
    if (M <= 0 || N <= 0 || K < 0) return 0;
    return static_cast<int>(candidates(Key{M, N, K, epi, out, aligned16 ? 1 : 0}).size());
}

int proj_num_candidates_hilo(int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16) {
    if (M <= 0 || N <= 0 || K < 0) return 0;
    return static_cast<int>(candidates(Key{M, N, 2 * K, epi, out, aligned16 ? 1 : 0, 1}).size());
}

proj_status proj_candidate_name_hilo(int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16, int index,
                                     char *buf, size_t len) {
    if (M <= 0 || N <= 0 || K < 0 || !buf) return PROJ_ERR_INVALID_ARG;
    std::vector<Candidate> c = candidates(Key{M, N, 2 * K, epi, out, aligned16 ? 1 : 0, 1});
    if (index < 0 || index >= static_cast<int>(c.size())) return PROJ_ERR_INVALID_ARG;
    if (c[index].name.size() + 1 > len) return PROJ_ERR_INVALID_ARG;
    std::strcpy(buf, c[index].name.c_str());
    return PROJ_OK;
}

proj_status proj_run_candidate_hilo(proj_ctx *ctx, int index, const void *X, const void *Whl, const void *bias,
                                    int epi, int64_t M, int64_t N, int64_t K, void *Y, int out, void *stream) {
    proj_status s = check_args(ctx, X, Whl, bias, epi, M, N, 2 * K, Y, out, 1);
    if (s != PROJ_OK || M == 0 || N == 0) return s;
    const Key k = make_key(X, Whl, epi, M, N, 2 * K, out, 1);
    std::vector<Candidate> c = candidates(k);
    if (index < 0 || index >= static_cast<int>(c.size())) {
        set_err(ctx, "candidate %d out of range (%d)", index, static_cast<int>(c.size()));
        return PROJ_ERR_INVALID_ARG;
    }
    if (!fits(c[index], k, ctx->ws_bytes)) return no_workspace(ctx, c[index], k);
    DeviceGuard g(ctx->device);
    hipError_t e = launch(c[index], make_args(ctx, X, Whl, bias, epi, M, N, 2 * K, Y, out, 1),
                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_candidate_name(int64_t M, int64_t N, int64_t K, int epi, int out, int aligned16, int index,
                                char *buf, size_t len) {
    if (M <= 0 || N <= 0 || K < 0 || !buf) return PROJ_ERR_INVALID_ARG;
    std::vector<Candidate> c = candidates(Key{M, N, K, epi, out, aligned16 ? 1 : 0});
    if (index < 0 || index >= static_cast<int>(c.size())) return PROJ_ERR_INVALID_ARG;
    if (c[index].name.size() + 1 > len) return PROJ_ERR_INVALID_ARG;
    std::strcpy(buf, c[index].name.c_str());
    return PROJ_OK;
}

proj_status proj_run_candidate(proj_ctx *ctx, int index, const void *X, const void *W, const void *bias, int epi,
                               int64_t M, int64_t N, int64_t K, void *Y, int out, void *stream) {
    proj_status s = check_args(ctx, X, W, bias, epi, M, N, K, Y, out);
    if (s != PROJ_OK || M == 0 || N == 0) return s;
    const Key k = make_key(X, W, epi, M, N, K, out);
    std::vector<Candidate> c = candidates(k);
    if (index < 0 || index >= static_cast<int>(c.size())) {
        set_err(ctx, "candidate %d out of range (%d)", index, static_cast<int>(c.size()));
        return PROJ_ERR_INVALID_ARG;
    }
    if (!fits(c[index], k, ctx->ws_bytes)) return no_workspace(ctx, c[index], k);
    DeviceGuard g(ctx->device);
    hipError_t e = launch(c[index], make_args(ctx, X, W, bias, epi, M, N, K, Y, out), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_get_plan_packed(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int tile16, int epi, int out,
                                 int aligned16, char *buf, size_t len) {
    return get_plan(ctx, Key{M, N, K, epi, out, aligned16 ? 1 : 0, 0, tile16}, buf, len);
}

int proj_num_candidates_packed(int64_t M, int64_t N, int64_t K, int tile16, int epi, int out, int aligned16) {
    if (M <= 0 || N <= 0 || K < 0 || !packable_tile(tile16)) return 0;
    return static_cast<int>(candidates(Key{M, N, K, epi, out, aligned16 ? 1 : 0, 0, tile16}).size());
}

proj_status proj_candidate_name_packed(int64_t M, int64_t N, int64_t K, int tile16, int epi, int out, int aligned16,
                                       int index, char *buf, size_t len) {
    if (M <= 0 || N <= 0 || K < 0 || !buf || !packable_tile(tile16)) return PROJ_ERR_INVALID_ARG;
    std::vector<Candidate> c = candidates(Key{M, N, K, epi, out, aligned16 ? 1 : 0, 0, tile16});
    if (index < 0 || index >= static_cast<int>(c.size())) return PROJ_ERR_INVALID_ARG;
    if (c[index].name.size() + 1 > len) return PROJ_ERR_INVALID_ARG;
    std::strcpy(buf, c[index].name.c_str());
    return PROJ_OK;
}

proj_status proj_run_candidate_packed(proj_ctx *ctx, int index, const void *X, const void *Wp, int tile16,
                                      const void *bias, int epi, int64_t M, int64_t N, int64_t K, void *Y, int out,
                                      void *stream) {
    proj_status s = check_args(ctx, X, Wp, bias, epi, M, N, K, Y, out, 0, tile16);
    if (s != PROJ_OK || M == 0 || N == 0) return s;
    if (!packable_tile(tile16)) return PROJ_ERR_INVALID_ARG;
    const Key k = make_key(X, Wp, epi, M, N, K, out, 0, tile16);
    std::vector<Candidate> c = candidates(k);
    if (index < 0 || index >= static_cast<int>(c.size())) {
        set_err(ctx, "candidate %d out of range (%d)", index, static_cast<int>(c.size()));
        return PROJ_ERR_INVALID_ARG;
    }
    if (!fits(c[index], k, ctx->ws_bytes)) return no_workspace(ctx, c[index], k);
    DeviceGuard g(ctx->device);
    hipError_t e = launch(c[index], make_args(ctx, X, Wp, bias, epi, M, N, K, Y, out, 0, tile16),
                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_read_probe(proj_ctx *ctx, const void *buf, size_t bytes, void *stream) {
    if (!ctx) return PROJ_ERR_INVALID_ARG;
    if (ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (ctx->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    if (bytes == 0) return PROJ_OK;
    if (!buf || reinterpret_cast<uintptr_t>(buf) % 16 || bytes % 16) {
        set_err(ctx, "read probe: buffer NULL, or buffer or size not a multiple of 16 bytes");
        return PROJ_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    unsigned *sink = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(ctx->zeros) + kZeroBytes);
    hipError_t e = launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(ctx, "launch", e);
    return PROJ_OK;
}

proj_status proj_graph_capture(proj_ctx *ctx, int n_calls, const void *const *X, const void *const *W,
                               const void *const *bias, void *const *Y, int epi, int64_t M, int64_t N, int64_t K,
                               int out, void *stream, proj_graph **graph) {
    if (!ctx || !graph || n_calls <= 0 || !X || !W || !Y || !stream) return PROJ_ERR_INVALID_ARG;
    if (ctx->magic == kDead) return PROJ_ERR_DESTROYED;
    if (ctx->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    *graph = nullptr;
    for (int i = 0; i < n_calls; ++i) {
        proj_status s = check_args(ctx, X[i], W[i], bias ? bias[i] : nullptr, epi, M, N, K, Y[i], out);
        if (s != PROJ_OK) return s;
    }
    if (M == 0 || N == 0) return PROJ_ERR_INVALID_ARG;  // nothing to capture
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (capturing(st)) {
        set_err(ctx, "stream is already capturing");
        return PROJ_ERR_INVALID_ARG;
    }
    DeviceGuard g(ctx->device);
    // plan first, outside capture (tunes on call 0's buffers)
    proj_status s = run_impl(ctx, X[0], W[0], bias ? bias[0] : nullptr, epi, M, N, K, Y[0], out, stream, false);
    if (s != PROJ_OK) return s;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(ctx, "hipStreamSynchronize", e);
    e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(ctx, "hipStreamBeginCapture", e);
    for (int i = 0; i < n_calls && s == PROJ_OK; ++i)
        s = run_impl(ctx, X[i], W[i], bias ? bias[i] : nullptr, epi, M, N, K, Y[i], out, stream, false);
    hipGraph_t gr = nullptr;
    e = hipStreamEndCapture(st, &gr);
    if (s != PROJ_OK) {
        if (gr) hipGraphDestroy(gr);
        return s;
    }
    if (e != hipSuccess) return hip_fail(ctx, "hipStreamEndCapture", e);
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, gr, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        hipGraphDestroy(gr);
        return hip_fail(ctx, "hipGraphInstantiate", e);
    }
    proj_graph *pg = new (std::nothrow) proj_graph{kMagic, ctx->device, ctx, gr, ex};
    if (!pg) {
        hipGraphExecDestroy(ex);
        hipGraphDestroy(gr);
        return PROJ_ERR_NO_MEMORY;
    }
    *graph = pg;
    return PROJ_OK;
}

proj_status proj_graph_launch(proj_graph *g, void *stream) {
    if (!g) return PROJ_ERR_INVALID_ARG;
    if (g->magic == kDead) return PROJ_ERR_DESTROYED;
    if (g->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    // the graph's kernels take the context's workspace and zero page: a
    // destroyed context's memory is gone (its struct stays as a marker)
    if (g->ctx->magic != kMagic) return PROJ_ERR_DESTROYED;
    DeviceGuard dg(g->device);
    if (hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) != hipSuccess) return PROJ_ERR_HIP;
    return PROJ_OK;
}

proj_status proj_graph_destroy(proj_graph *g) {
    if (!g) return PROJ_ERR_INVALID_ARG;
    if (g->magic == kDead) return PROJ_ERR_DESTROYED;
    if (g->magic != kMagic) return PROJ_ERR_INVALID_ARG;
    DeviceGuard dg(g->device);
    hipGraphExecDestroy(g->exec);
    hipGraphDestroy(g->graph);
    // kept allocated as a marker (see proj_destroy)
    g->exec = nullptr;
    g->graph = nullptr;
    g->magic = kDead;
    return PROJ_OK;
}

}  // extern "C"
