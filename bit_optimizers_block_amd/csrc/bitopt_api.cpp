// bitopt_api.cpp -- the C ABI of libbitopt (declared in include/bitopt.h):
// argument checks, per-step scalars, the host codebook builder and kernel dispatch.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "bitopt.h"
#include "dynamic_map.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return BITOPT_OK;
}

int device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(BITOPT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dtype(int32_t d) { return d == BITOPT_F32 || d == BITOPT_F16 || d == BITOPT_BF16; }
bool valid_blocksize(int32_t b) { return b == 256 || b == 2048; }
int elem_size(int32_t d) { return d == BITOPT_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool beta_ok(float b) { return b >= 0.0f && b < 1.0f; }

// Hyper-parameter checks shared by every step entry point.
int check_hparams(const bitopt_hparams* hp, int32_t step, int64_t n, const char* fn) {
    if (!hp) return fail(BITOPT_ERR_INVALID_ARG, "%s: hp is NULL", fn);
    if (hp->optimizer < BITOPT_ADAM || hp->optimizer > BITOPT_ADAGRAD)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown optimizer %d", fn, hp->optimizer);
    if (step < 1) return fail(BITOPT_ERR_INVALID_ARG, "%s: step must be >= 1 (got %d)", fn, step);
    if (n < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: n < 0", fn);
    if (!valid_blocksize(hp->blocksize))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: blocksize must be 256 or 2048 (got %d)", fn, hp->blocksize);
    if (!beta_ok(hp->beta1) || !beta_ok(hp->beta2))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: betas must lie in [0, 1)", fn);
    if (hp->optimizer == BITOPT_ADEMAMIX && !beta_ok(hp->beta3))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: beta3 must lie in [0, 1)", fn);
    if (hp->optimizer == BITOPT_ADEMAMIX && hp->t_beta3 > 0 && !(hp->beta1 > 0.0f && hp->beta3 > 0.0f))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: a beta3 schedule needs beta1 > 0 and beta3 > 0", fn);
    if (!(hp->eps >= 0.0f)) return fail(BITOPT_ERR_INVALID_ARG, "%s: eps < 0", fn);
    if (!(hp->lr >= 0.0f)) return fail(BITOPT_ERR_INVALID_ARG, "%s: lr < 0", fn);
    if (!(hp->max_unorm >= 0.0f)) return fail(BITOPT_ERR_INVALID_ARG, "%s: max_unorm < 0", fn);
    if (!std::isfinite(hp->weight_decay) || !std::isfinite(hp->alpha))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: weight_decay and alpha must be finite", fn);
    return BITOPT_OK;
}

// beta3(t) of AdEMAMix: the slow EMA's half-life grows linearly in t from beta1's
// to beta3's over T steps (1/ln beta3(t) interpolates 1/ln beta1 and 1/ln beta3),
// capped at beta3.
double beta3_at(double b1, double b3, int32_t t, int32_t T) {
    if (T <= 0) return b3;
    const double l1 = std::log(b1), l3 = std::log(b3);
    const double f = (double)t / (double)T;
    const double v = std::exp(l1 * l3 / ((1.0 - f) * l3 + f * l1));
    return std::min(v, b3);
}

double alpha_at(double alpha, int32_t t, int32_t T) {
    if (T <= 0) return alpha;
    return alpha * std::min((double)t / (double)T, 1.0);
}

bitopt::StepScalars make_scalars(const bitopt_hparams& h, int32_t t) {
    bitopt::StepScalars s{};
    const double b1 = h.beta1, b2 = h.beta2;
    s.lr = h.lr; s.b1 = h.beta1; s.b2 = h.beta2; s.eps = h.eps; s.wd = h.weight_decay;
    s.omb1 = (float)(1.0 - b1);
    s.omb2 = (float)(1.0 - b2);
    s.ic1 = (float)(1.0 / (1.0 - std::pow(b1, (double)t)));
    s.rs2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)t)));
    s.decay = (float)(1.0 - (double)h.lr * (double)h.weight_decay);
    const double b3t = beta3_at(b1, (double)h.beta3, t, h.t_beta3);
    s.b3t = (float)b3t;
    s.omb3 = (float)(1.0 - b3t);
    s.alpha_t = (float)alpha_at((double)h.alpha, t, h.t_alpha);
    s.max_unorm = h.max_unorm;
    // the exact product of the two fp32 scalars, rounded once
    s.lric1 = (float)((double)s.lr * (double)s.ic1);
    // the root optimizers' denominator then stays below 2^85, so its hardware
    // reciprocal is a normal number, and the folded numerator scale carries one
    // rounding (the error bound of the 16-bit parameter path)
    const bool lric1_ok = s.lric1 == 0.0f || (std::isfinite(s.lric1) && s.lric1 >= 0x1p-126f);
    s.fast_root = (h.eps <= 0x1p60f && s.rs2 <= 0x1p20f && lric1_ok) ? 1 : 0;
    return s;
}

}  // namespace

namespace bitopt {

// Compute units of each device, queried on first use.  Default groups per CU: 256
// 4-wave groups, i.e. one tile per wave up to 64 M elements (B = 256) on 256 CUs, and
// a grid stride beyond that, so very large launches stage the LDS codebooks once per
// group for several tiles rather than once per tile.  Measured on MI355X: one tile
// per wave streams best for most steps (the hardware refills CUs as groups retire).
// Launches that pass resident_per_cu (see step_dispatch.h) use that many groups per
// CU instead: a grid resident at once, or the multi-tensor launches' 512.
int64_t group_cap(int resident_per_cu) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cus[kMaxDev];
    static const int env_per_cu = [] {
        const char* e = std::getenv("BITOPT_GROUPS_PER_CU");
        const int v = e ? std::atoi(e) : 0;
        return v > 0 ? v : 0;
    }();
    const int per_cu = env_per_cu > 0 ? env_per_cu : (resident_per_cu > 0 ? resident_per_cu : 256);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 2048;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return (int64_t)c * per_cu;
}

int resident_groups_per_cu(const void* kernel) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

}  // namespace bitopt

namespace {

hipError_t dispatch_step(const bitopt::StepArgs& a, int opt, int dtype, int bs, bool quant, bool skip,
                         bool unorm, hipStream_t s) {
    switch (opt) {
    case BITOPT_ADAM: return bitopt::launch_step_adam(a, dtype, bs, quant, skip, unorm, s);
    case BITOPT_ADEMAMIX: return bitopt::launch_step_ademamix(a, dtype, bs, quant, skip, unorm, s);
    case BITOPT_MOMENTUM: return bitopt::launch_step_momentum(a, dtype, bs, quant, skip, unorm, s);
    case BITOPT_RMSPROP: return bitopt::launch_step_rmsprop(a, dtype, bs, quant, skip, unorm, s);
    case BITOPT_ADAGRAD: return bitopt::launch_step_adagrad(a, dtype, bs, quant, skip, unorm, s);
    default: return bitopt::launch_step_lion(a, dtype, bs, quant, skip, unorm, s);
    }
}

// Elements per wave tile of the step kernels.
int64_t tile_elems(int32_t blocksize) {
    return blocksize == 256 ? bitopt::Layout<256>::TE : bitopt::Layout<2048>::TE;
}

bool vec_ok(const bitopt_hparams* hp, const void* p, const void* g, int32_t dtype, int64_t n,
            const void* s1, const void* s2) {
    const int es = elem_size(dtype);
    bool vec = aligned(p, 4 * es) && aligned(g, 4 * es) && aligned(s1, 16) && (!s2 || aligned(s2, 16));
    if (hp->optimizer == BITOPT_ADEMAMIX) vec = vec && (n % 16 == 0);
    return vec;
}

int run_step(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype, int64_t n,
             void* s1, void* s2, float* a1, float* a2, const float* q1, const float* q2, bool quant,
             void* stream, const char* fn) {
    bitopt::StepArgs a{};
    a.p = p; a.g = g; a.s1 = s1; a.s2 = s2; a.a1 = a1; a.a2 = a2; a.q1 = q1; a.q2 = q2;
    a.n = n;
    a.nb = (n + hp->blocksize - 1) / hp->blocksize;
    a.s = make_scalars(*hp, step);
    a.vec = vec_ok(hp, p, g, dtype, n, s1, s2) ? 1 : 0;
    hipError_t e = dispatch_step(a, hp->optimizer, dtype, hp->blocksize, quant, hp->skip_zeros != 0,
                                 hp->max_unorm > 0.0f, reinterpret_cast<hipStream_t>(stream));
    return device_status(e, fn);
}

}  // namespace

extern "C" {

const char* bitopt_last_error(void) { return g_last_error.c_str(); }

int32_t bitopt_abi_version(void) { return 1; }

int bitopt_create_dynamic_map(int is_signed, float* out256) {
    if (!out256) return fail(BITOPT_ERR_INVALID_ARG, "bitopt_create_dynamic_map: out256 is NULL");
    bitopt::build_dynamic_map(is_signed != 0, out256);
    return ok();
}

int bitopt_step_scalars(const bitopt_hparams* hp, int32_t step, float* out14) {
    if (!out14) return fail(BITOPT_ERR_INVALID_ARG, "bitopt_step_scalars: out14 is NULL");
    if (int rc = check_hparams(hp, step, 0, "bitopt_step_scalars")) return rc;
    const bitopt::StepScalars s = make_scalars(*hp, step);
    const float v[14] = {s.lr, s.b1, s.b2, s.eps, s.wd, s.omb1, s.omb2, s.ic1, s.rs2, s.decay,
                         s.b3t, s.omb3, s.alpha_t, s.max_unorm};
    std::memcpy(out14, v, sizeof v);
    return ok();
}

int bitopt_quantize_blockwise(const void* x, int32_t dtype, int64_t n, const float* qmap, int32_t blocksize,
                              uint8_t* codes, float* absmax, void* stream) {
    const char* fn = "bitopt_quantize_blockwise";
    if (n < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: n < 0", fn);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (!valid_blocksize(blocksize)) return fail(BITOPT_ERR_INVALID_ARG, "%s: blocksize must be 256 or 2048", fn);
    if (n == 0) return ok();
    if (!x || !qmap || !codes || !absmax) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    bitopt::CodecArgs a{};
    a.x = x; a.codes = codes; a.absmax = absmax; a.qmap = qmap; a.n = n;
    a.nb = (n + blocksize - 1) / blocksize;
    a.vec = (aligned(x, 4 * elem_size(dtype)) && aligned(codes, 16)) ? 1 : 0;
    return device_status(bitopt::launch_quantize(a, dtype, blocksize, reinterpret_cast<hipStream_t>(stream)), fn);
}

int bitopt_dequantize_blockwise(const uint8_t* codes, const float* absmax, const float* qmap, int64_t n,
                                int32_t blocksize, void* out, int32_t dtype, void* stream) {
    const char* fn = "bitopt_dequantize_blockwise";
    if (n < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: n < 0", fn);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (!valid_blocksize(blocksize)) return fail(BITOPT_ERR_INVALID_ARG, "%s: blocksize must be 256 or 2048", fn);
    if (n == 0) return ok();
    if (!codes || !absmax || !qmap || !out) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    bitopt::CodecArgs a{};
    a.out = out; a.codes = const_cast<uint8_t*>(codes); a.absmax = const_cast<float*>(absmax); a.qmap = qmap;
    a.n = n;
    a.nb = (n + blocksize - 1) / blocksize;
    a.vec = (aligned(out, 4 * elem_size(dtype)) && aligned(codes, 4)) ? 1 : 0;
    return device_status(bitopt::launch_dequantize(a, dtype, blocksize, reinterpret_cast<hipStream_t>(stream)), fn);
}

int bitopt_step_8bit_blockwise_2state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                      int32_t dtype, int64_t n, uint8_t* state1, uint8_t* state2,
                                      float* absmax1, float* absmax2, const float* qmap1,
                                      const float* qmap2, void* stream) {
    const char* fn = "bitopt_step_8bit_blockwise_2state";
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (hp->optimizer != BITOPT_ADAM && hp->optimizer != BITOPT_ADEMAMIX)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: optimizer %d is not a 2-state optimizer", fn, hp->optimizer);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (n == 0) return ok();
    if (!p || !g || !state1 || !state2 || !absmax1 || !absmax2 || !qmap1 || !qmap2)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    return run_step(hp, step, p, g, dtype, n, state1, state2, absmax1, absmax2, qmap1, qmap2, true, stream, fn);
}

int bitopt_step_8bit_blockwise_1state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                      int32_t dtype, int64_t n, uint8_t* state1, float* absmax1,
                                      const float* qmap1, void* stream) {
    const char* fn = "bitopt_step_8bit_blockwise_1state";
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (hp->optimizer != BITOPT_MOMENTUM && hp->optimizer != BITOPT_LION && hp->optimizer != BITOPT_RMSPROP &&
        hp->optimizer != BITOPT_ADAGRAD)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: optimizer %d is not a 1-state optimizer", fn, hp->optimizer);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (n == 0) return ok();
    if (!p || !g || !state1 || !absmax1 || !qmap1) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    return run_step(hp, step, p, g, dtype, n, state1, nullptr, absmax1, nullptr, qmap1, nullptr, true, stream, fn);
}

int bitopt_step_32bit_2state(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype,
                             int64_t n, float* state1, float* state2, void* stream) {
    const char* fn = "bitopt_step_32bit_2state";
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (hp->optimizer != BITOPT_ADAM && hp->optimizer != BITOPT_ADEMAMIX)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: optimizer %d is not a 2-state optimizer", fn, hp->optimizer);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (n == 0) return ok();
    if (!p || !g || !state1 || !state2) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    return run_step(hp, step, p, g, dtype, n, state1, state2, nullptr, nullptr, nullptr, nullptr, false, stream, fn);
}

int bitopt_step_32bit_1state(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype,
                             int64_t n, float* state1, void* stream) {
    const char* fn = "bitopt_step_32bit_1state";
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (hp->optimizer != BITOPT_MOMENTUM && hp->optimizer != BITOPT_LION && hp->optimizer != BITOPT_RMSPROP &&
        hp->optimizer != BITOPT_ADAGRAD)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: optimizer %d is not a 1-state optimizer", fn, hp->optimizer);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (n == 0) return ok();
    if (!p || !g || !state1) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    return run_step(hp, step, p, g, dtype, n, state1, nullptr, nullptr, nullptr, nullptr, nullptr, false, stream, fn);
}

int bitopt_host_state_alloc(int64_t bytes, void** ptr) {
    const char* fn = "bitopt_host_state_alloc";
    if (!ptr || bytes <= 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: bytes must be > 0 and ptr non-NULL", fn);
    *ptr = nullptr;
    void* h = nullptr;
    hipError_t e = hipHostMalloc(&h, (size_t)bytes, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return device_status(e, fn);
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess || d != h) {
        (void)hipHostFree(h);
        if (e != hipSuccess) return device_status(e, fn);
        return fail(BITOPT_ERR_UNSUPPORTED, "%s: the device address of pinned host memory differs from its host address", fn);
    }
    *ptr = h;
    return ok();
}

int bitopt_host_state_free(void* ptr) {
    if (!ptr) return ok();
    return device_status(hipHostFree(ptr), "bitopt_host_state_free");
}

int64_t bitopt_tensorwise_workspace_bytes(void) { return (int64_t)bitopt::tensorwise_workspace_words() * 4; }

}  // extern "C"

namespace {

// ---------------------------------------------------------------- paged (staged) state

constexpr int64_t kPageQuantum = 4096;     // chunk sizes are multiples of this many elements
constexpr int64_t kStageAlign = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Layout of one staging buffer for chunks of C elements: the chunk's codes and absmax
// in the order and shape a step call takes them.
struct StageLayout {
    int64_t s1, s2, a1, a2, bytes;   // offsets and total bytes
};

StageLayout stage_layout(int optimizer, int32_t blocksize, int64_t C) {
    const bool two = optimizer == BITOPT_ADAM || optimizer == BITOPT_ADEMAMIX;
    const int64_t k1 = optimizer == BITOPT_ADEMAMIX ? 2 : 1;
    const int64_t nbc = (C + blocksize - 1) / blocksize;
    StageLayout L{};
    int64_t off = 0;
    L.s1 = off; off = align_up(off + k1 * C, kStageAlign);
    L.s2 = off; off = two ? align_up(off + C, kStageAlign) : off;
    L.a1 = off; off = align_up(off + 4 * k1 * nbc, kStageAlign);
    L.a2 = off; off = two ? align_up(off + 4 * nbc, kStageAlign) : off;
    L.bytes = off;
    return L;
}

// Events of the staged step, per device and per calling thread: one call enqueues
// all of its work before it returns, and a stream wait binds to the record made
// before it, so later calls can re-record them.
struct StageEvents {
    hipEvent_t start, in[2], comp[2], out[2];
    bool ready;
};

hipError_t stage_events(StageEvents** out) {
    constexpr int kMaxDev = 64;
    thread_local StageEvents pool[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    StageEvents& E = pool[dev];
    if (!E.ready) {
        hipEvent_t* all[7] = {&E.start, &E.in[0], &E.in[1], &E.comp[0], &E.comp[1], &E.out[0], &E.out[1]};
        for (hipEvent_t* ev : all) {
            e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        E.ready = true;
    }
    *out = &E;
    return hipSuccess;
}

}  // namespace

extern "C" {

int64_t bitopt_paged_staging_bytes(const bitopt_hparams* hp, int64_t chunk_elems) {
    if (!hp || chunk_elems < 1 || !valid_blocksize(hp->blocksize) || hp->optimizer < BITOPT_ADAM ||
        hp->optimizer > BITOPT_ADAGRAD)
        return -1;
    return 2 * stage_layout(hp->optimizer, hp->blocksize, align_up(chunk_elems, kPageQuantum)).bytes;
}

int bitopt_step_8bit_paged(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype,
                           int64_t n, uint8_t* host_state1, uint8_t* host_state2, float* host_absmax1,
                           float* host_absmax2, const float* qmap1, const float* qmap2, void* staging,
                           int64_t staging_bytes, void* h2d_stream, void* d2h_stream, void* stream) {
    const char* fn = "bitopt_step_8bit_paged";
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    if (n == 0) return ok();
    if (!p || !g || !host_state1 || !host_absmax1 || !qmap1 || !staging ||
        (two && (!host_state2 || !host_absmax2 || !qmap2)))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(staging, kStageAlign)) return fail(BITOPT_ERR_INVALID_ARG, "%s: staging not 256-byte aligned", fn);
    if (h2d_stream == d2h_stream || h2d_stream == stream || d2h_stream == stream)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: the two copy streams and the step stream must be distinct", fn);
    // the largest chunk (a multiple of kPageQuantum elements) whose two buffers fit
    const int64_t B = hp->blocksize;
    int64_t C = align_up(n, kPageQuantum);
    while (C > kPageQuantum && 2 * stage_layout(hp->optimizer, hp->blocksize, C).bytes > staging_bytes)
        C = std::max(kPageQuantum, (C / 2) / kPageQuantum * kPageQuantum);
    const StageLayout L = stage_layout(hp->optimizer, hp->blocksize, C);
    if (2 * L.bytes > staging_bytes)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: staging of %lld bytes is below the minimum %lld", fn,
                    (long long)staging_bytes, (long long)(2 * L.bytes));
    StageEvents* E = nullptr;
    if (hipError_t e = stage_events(&E); e != hipSuccess) return device_status(e, fn);
    hipStream_t sh = reinterpret_cast<hipStream_t>(h2d_stream), sd = reinterpret_cast<hipStream_t>(d2h_stream),
                sc = reinterpret_cast<hipStream_t>(stream);
    const int64_t k1 = hp->optimizer == BITOPT_ADEMAMIX ? 2 : 1;
    const int64_t nb = (n + B - 1) / B;
    const int es = elem_size(dtype);
    uint8_t* base = static_cast<uint8_t*>(staging);
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    // nothing of this call reads the host state before the work already on `stream`
    // (earlier steps and their write-backs) is complete
    chk(hipEventRecord(E->start, sc));
    chk(hipStreamWaitEvent(sh, E->start, 0));
    const int64_t nchunks = (n + C - 1) / C;
    for (int64_t i = 0; i < nchunks && e == hipSuccess; ++i) {
        const int b = (int)(i & 1);
        const int64_t c0 = i * C, len = std::min(C, n - c0);
        const int64_t cb0 = c0 / B, nbc = (len + B - 1) / B;
        uint8_t* buf = base + b * L.bytes;
        uint8_t* ds1 = buf + L.s1;
        uint8_t* ds2 = buf + L.s2;
        float* da1 = reinterpret_cast<float*>(buf + L.a1);
        float* da2 = reinterpret_cast<float*>(buf + L.a2);
        if (i >= 2) chk(hipStreamWaitEvent(sh, E->out[b], 0));     // buffer b written back
        for (int64_t k = 0; k < k1; ++k) {
            chk(hipMemcpyAsync(ds1 + k * len, host_state1 + k * n + c0, len, hipMemcpyHostToDevice, sh));
            chk(hipMemcpyAsync(da1 + k * nbc, host_absmax1 + k * nb + cb0, 4 * nbc, hipMemcpyHostToDevice, sh));
        }
        if (two) {
            chk(hipMemcpyAsync(ds2, host_state2 + c0, len, hipMemcpyHostToDevice, sh));
            chk(hipMemcpyAsync(da2, host_absmax2 + cb0, 4 * nbc, hipMemcpyHostToDevice, sh));
        }
        chk(hipEventRecord(E->in[b], sh));
        chk(hipStreamWaitEvent(sc, E->in[b], 0));
        if (e != hipSuccess) break;
        if (int rc = run_step(hp, step, static_cast<uint8_t*>(p) + c0 * es, static_cast<const uint8_t*>(g) + c0 * es,
                              dtype, len, ds1, two ? ds2 : nullptr, da1, two ? da2 : nullptr, qmap1,
                              two ? qmap2 : nullptr, true, stream, fn))
            return rc;
        chk(hipEventRecord(E->comp[b], sc));
        chk(hipStreamWaitEvent(sd, E->comp[b], 0));
        for (int64_t k = 0; k < k1; ++k) {
            chk(hipMemcpyAsync(host_state1 + k * n + c0, ds1 + k * len, len, hipMemcpyDeviceToHost, sd));
            chk(hipMemcpyAsync(host_absmax1 + k * nb + cb0, da1 + k * nbc, 4 * nbc, hipMemcpyDeviceToHost, sd));
        }
        if (two) {
            chk(hipMemcpyAsync(host_state2 + c0, ds2, len, hipMemcpyDeviceToHost, sd));
            chk(hipMemcpyAsync(host_absmax2 + cb0, da2, 4 * nbc, hipMemcpyDeviceToHost, sd));
        }
        chk(hipEventRecord(E->out[b], sd));
    }
    // the step stream completes only after every write-back (they run in order on d2h)
    chk(hipStreamWaitEvent(sc, E->out[(nchunks - 1) & 1], 0));
    return device_status(e, fn);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- paged state, cached in an HBM page pool

// One frame of the pool: room for one page (the state of page_elems elements of one
// tensor, in the staging layout), the identity of the page it holds and the events
// that order its copies and steps.
struct PoolFrame {
    const uint8_t* key = nullptr;      // host_state1 of the owning tensor (nullptr: free)
    int64_t page = 0;                  // page index inside that tensor
    uint8_t* hs1 = nullptr;            // the owner's host buffers and size (write-back targets)
    uint8_t* hs2 = nullptr;
    float* ha1 = nullptr;
    float* ha2 = nullptr;
    int64_t n = 0;
    bool dirty = false;                // stepped since it was copied in or last written back
    uint64_t tick = 0;                 // last use (least recently used frame is evicted first)
    hipStream_t last_stream = nullptr; // stream of its last step
    hipEvent_t in = nullptr;           // copy-in complete
    hipEvent_t comp = nullptr;         // last step on it complete
    bool stepped = false;              // comp has been recorded
    bool wb_pending = false;           // written back since its last step; a step must first wait for tail
};

struct PageKeyHash {
    size_t operator()(const std::pair<const uint8_t*, int64_t>& k) const {
        return std::hash<const void*>()(k.first) ^ (std::hash<int64_t>()(k.second) * 0x9E3779B97F4A7C15ull);
    }
};

}  // namespace

struct bitopt_page_pool {
    int device = 0;
    int32_t optimizer = 0, blocksize = 0;
    int64_t C = 0;                     // page size in elements
    StageLayout L{};
    uint8_t* frames = nullptr;
    std::vector<PoolFrame> fr;
    std::unordered_map<std::pair<const uint8_t*, int64_t>, int, PageKeyHash> where;
    hipStream_t h2d = nullptr, d2h = nullptr;   // the pool's own copy streams (default priority)
    hipEvent_t tail = nullptr;                  // recorded on d2h after every write-back
    uint64_t tail_seq = 0, h2d_seen = 0;        // records of tail; the last one h2d waited for
    hipEvent_t start = nullptr;
    uint64_t tick = 0;
    int64_t page_ins = 0, write_backs = 0, hits = 0;
};

namespace {

int pool_device_ok(const bitopt_page_pool* pool, const char* fn) {
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return device_status(e, fn);
    if (dev != pool->device)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: the pool was created on device %d, the current device is %d", fn,
                    pool->device, dev);
    return BITOPT_OK;
}

// Enqueues the write-back of frame f's page to its owner's host buffers on the pool's
// d2h stream (after the frame's last step, when that ran on a stream other than
// `after`, whose own order the caller has already joined to d2h).
hipError_t pool_write_back(bitopt_page_pool* pool, PoolFrame& F, hipStream_t after) {
    const int64_t B = pool->blocksize, C = pool->C;
    const bool two = pool->optimizer == BITOPT_ADAM || pool->optimizer == BITOPT_ADEMAMIX;
    const int64_t k1 = pool->optimizer == BITOPT_ADEMAMIX ? 2 : 1;
    const int64_t c0 = F.page * C, len = std::min(C, F.n - c0);
    const int64_t nb = (F.n + B - 1) / B, cb0 = c0 / B, nbc = (len + B - 1) / B;
    uint8_t* buf = pool->frames + (&F - pool->fr.data()) * pool->L.bytes;
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    if (F.last_stream != after) chk(hipStreamWaitEvent(pool->d2h, F.comp, 0));
    for (int64_t k = 0; k < k1; ++k) {
        chk(hipMemcpyAsync(F.hs1 + k * F.n + c0, buf + pool->L.s1 + k * len, len, hipMemcpyDeviceToHost, pool->d2h));
        chk(hipMemcpyAsync(F.ha1 + k * nb + cb0, buf + pool->L.a1 + 4 * k * nbc, 4 * nbc, hipMemcpyDeviceToHost,
                           pool->d2h));
    }
    if (two) {
        chk(hipMemcpyAsync(F.hs2 + c0, buf + pool->L.s2, len, hipMemcpyDeviceToHost, pool->d2h));
        chk(hipMemcpyAsync(F.ha2 + cb0, buf + pool->L.a2, 4 * nbc, hipMemcpyDeviceToHost, pool->d2h));
    }
    F.dirty = false;
    F.wb_pending = true;
    ++pool->write_backs;
    return e;
}

}  // namespace

extern "C" {

int64_t bitopt_page_pool_frame_bytes(const bitopt_hparams* hp, int64_t page_elems) {
    if (!hp || page_elems < 1 || page_elems % kPageQuantum != 0 || !valid_blocksize(hp->blocksize) ||
        hp->optimizer < BITOPT_ADAM || hp->optimizer > BITOPT_ADAGRAD)
        return -1;
    return stage_layout(hp->optimizer, hp->blocksize, page_elems).bytes;
}

int bitopt_page_pool_create(const bitopt_hparams* hp, int64_t page_elems, void* frames, int64_t frames_bytes,
                            bitopt_page_pool** pool) {
    const char* fn = "bitopt_page_pool_create";
    if (!pool) return fail(BITOPT_ERR_INVALID_ARG, "%s: pool is NULL", fn);
    *pool = nullptr;
    if (int rc = check_hparams(hp, 1, 0, fn)) return rc;
    if (page_elems < kPageQuantum || page_elems % kPageQuantum != 0)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: page_elems must be a positive multiple of %lld (got %lld)", fn,
                    (long long)kPageQuantum, (long long)page_elems);
    if (!frames) return fail(BITOPT_ERR_INVALID_ARG, "%s: frames is NULL", fn);
    if (!aligned(frames, kStageAlign)) return fail(BITOPT_ERR_INVALID_ARG, "%s: frames not 256-byte aligned", fn);
    const StageLayout L = stage_layout(hp->optimizer, hp->blocksize, page_elems);
    const int64_t nframes = frames_bytes / L.bytes;
    if (nframes < 2)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: %lld bytes hold %lld frames of %lld bytes; at least 2 are needed", fn,
                    (long long)frames_bytes, (long long)nframes, (long long)L.bytes);
    if (nframes > (int64_t)1 << 20) return fail(BITOPT_ERR_INVALID_ARG, "%s: more than 2^20 frames", fn);
    auto* P = new bitopt_page_pool;
    P->optimizer = hp->optimizer;
    P->blocksize = hp->blocksize;
    P->C = page_elems;
    P->L = L;
    P->frames = static_cast<uint8_t*>(frames);
    P->fr.resize((size_t)nframes);
    hipError_t e = hipGetDevice(&P->device);
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    chk(hipStreamCreateWithFlags(&P->h2d, hipStreamNonBlocking));
    chk(hipStreamCreateWithFlags(&P->d2h, hipStreamNonBlocking));
    chk(hipEventCreateWithFlags(&P->tail, hipEventDisableTiming));
    chk(hipEventCreateWithFlags(&P->start, hipEventDisableTiming));
    for (PoolFrame& F : P->fr) {
        chk(hipEventCreateWithFlags(&F.in, hipEventDisableTiming));
        chk(hipEventCreateWithFlags(&F.comp, hipEventDisableTiming));
    }
    if (e != hipSuccess) {
        (void)bitopt_page_pool_destroy(P);
        return device_status(e, fn);
    }
    *pool = P;
    return ok();
}

int bitopt_page_pool_destroy(bitopt_page_pool* pool) {
    if (!pool) return ok();
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    // the pool's copies may still read or write frames and host buffers
    if (pool->h2d) chk(hipStreamSynchronize(pool->h2d));
    if (pool->d2h) chk(hipStreamSynchronize(pool->d2h));
    for (PoolFrame& F : pool->fr) {
        if (F.comp && F.stepped) chk(hipEventSynchronize(F.comp));
        if (F.in) chk(hipEventDestroy(F.in));
        if (F.comp) chk(hipEventDestroy(F.comp));
    }
    if (pool->tail) chk(hipEventDestroy(pool->tail));
    if (pool->start) chk(hipEventDestroy(pool->start));
    if (pool->h2d) chk(hipStreamDestroy(pool->h2d));
    if (pool->d2h) chk(hipStreamDestroy(pool->d2h));
    delete pool;
    return device_status(e, "bitopt_page_pool_destroy");
}

int bitopt_step_8bit_pooled(bitopt_page_pool* pool, const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                            int32_t dtype, int64_t n, uint8_t* host_state1, uint8_t* host_state2,
                            float* host_absmax1, float* host_absmax2, const float* qmap1, const float* qmap2,
                            void* stream) {
    const char* fn = "bitopt_step_8bit_pooled";
    if (!pool) return fail(BITOPT_ERR_INVALID_ARG, "%s: pool is NULL", fn);
    if (int rc = check_hparams(hp, step, n, fn)) return rc;
    if (hp->optimizer != pool->optimizer || hp->blocksize != pool->blocksize)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: the pool holds optimizer %d, blocksize %d state (got %d, %d)", fn,
                    pool->optimizer, pool->blocksize, hp->optimizer, hp->blocksize);
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    if (n == 0) return ok();
    if (!p || !g || !host_state1 || !host_absmax1 || !qmap1 || (two && (!host_state2 || !host_absmax2 || !qmap2)))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!two) { host_state2 = nullptr; host_absmax2 = nullptr; }
    if (int rc = pool_device_ok(pool, fn)) return rc;
    const int64_t C = pool->C, B = hp->blocksize;
    const int64_t npages = (n + C - 1) / C;
    // every page of this tensor already in the pool must belong to the same buffers
    for (int64_t i = 0; i < npages; ++i) {
        auto it = pool->where.find({host_state1, i});
        if (it == pool->where.end()) continue;
        const PoolFrame& F = pool->fr[(size_t)it->second];
        if (F.n != n || F.hs2 != host_state2 || F.ha1 != host_absmax1 || F.ha2 != host_absmax2)
            return fail(BITOPT_ERR_INVALID_ARG,
                        "%s: host_state1 is in the pool with other companion buffers or size; flush with evict first",
                        fn);
    }
    hipStream_t sc = reinterpret_cast<hipStream_t>(stream);
    const int64_t k1 = hp->optimizer == BITOPT_ADEMAMIX ? 2 : 1;
    const int64_t nb = (n + B - 1) / B;
    const int es = elem_size(dtype);
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    const uint64_t call_start = pool->tick + 1;   // frames stepped by this call have tick >= call_start
    // At the first page that is not resident, `start` is recorded on sc: the copy-in stream
    // waits for it (host state written by work already on sc, e.g. another pool's flush, is
    // read only after it) and so does the write-back stream (pages stepped on sc so far).
    bool started = false, h2d_joined = false, d2h_joined = false;
    bool waited_tail = false;               // sc ordered after every write-back enqueued so far
    auto start = [&]() {
        if (!started) {
            chk(hipEventRecord(pool->start, sc));
            started = true;
        }
    };
    for (int64_t i = 0; i < npages && e == hipSuccess; ++i) {
        const int64_t c0 = i * C, len = std::min(C, n - c0);
        const int64_t cb0 = c0 / B, nbc = (len + B - 1) / B;
        int f;
        auto it = pool->where.find({host_state1, i});
        if (it != pool->where.end()) {
            f = it->second;
            PoolFrame& F = pool->fr[(size_t)f];
            if (F.last_stream != sc) chk(hipStreamWaitEvent(sc, F.comp, 0));
            if (F.wb_pending) {              // a flush's write-back may still read the frame
                if (!waited_tail) chk(hipStreamWaitEvent(sc, pool->tail, 0));
                waited_tail = true;
                F.wb_pending = false;
            }
            ++pool->hits;
        } else {
            // a free frame, else the least recently used one (pages this call has stepped
            // are the most recent, so they go last)
            f = -1;
            for (size_t j = 0; j < pool->fr.size(); ++j) {
                const PoolFrame& F = pool->fr[j];
                if (!F.key) { f = (int)j; break; }
                if (f < 0 || F.tick < pool->fr[(size_t)f].tick) f = (int)j;
            }
            PoolFrame& F = pool->fr[(size_t)f];
            start();
            if (F.key) {
                if (F.dirty) {
                    if (!d2h_joined) {     // one wait covers every earlier step on sc
                        chk(hipStreamWaitEvent(pool->d2h, pool->start, 0));
                        d2h_joined = true;
                    }
                    if (F.last_stream == sc && F.tick >= call_start) {
                        // stepped in this call, possibly after `start`: wait for that step itself
                        chk(hipStreamWaitEvent(pool->d2h, F.comp, 0));
                    }
                    chk(pool_write_back(pool, F, sc));
                    chk(hipEventRecord(pool->tail, pool->d2h));
                    ++pool->tail_seq;
                }
                pool->where.erase({F.key, F.page});
                F.key = nullptr;
            }
            uint8_t* buf = pool->frames + (int64_t)f * pool->L.bytes;
            if (!h2d_joined) {
                chk(hipStreamWaitEvent(pool->h2d, pool->start, 0));
                h2d_joined = true;
            }
            // the host copy is current only once every write-back enqueued so far is done
            if (pool->h2d_seen != pool->tail_seq) {
                chk(hipStreamWaitEvent(pool->h2d, pool->tail, 0));
                pool->h2d_seen = pool->tail_seq;
            }
            for (int64_t k = 0; k < k1; ++k) {
                chk(hipMemcpyAsync(buf + pool->L.s1 + k * len, host_state1 + k * n + c0, len, hipMemcpyHostToDevice,
                                   pool->h2d));
                chk(hipMemcpyAsync(buf + pool->L.a1 + 4 * k * nbc, host_absmax1 + k * nb + cb0, 4 * nbc,
                                   hipMemcpyHostToDevice, pool->h2d));
            }
            if (two) {
                chk(hipMemcpyAsync(buf + pool->L.s2, host_state2 + c0, len, hipMemcpyHostToDevice, pool->h2d));
                chk(hipMemcpyAsync(buf + pool->L.a2, host_absmax2 + cb0, 4 * nbc, hipMemcpyHostToDevice, pool->h2d));
            }
            chk(hipEventRecord(F.in, pool->h2d));
            chk(hipStreamWaitEvent(sc, F.in, 0));
            F.key = host_state1;
            F.page = i;
            F.hs1 = host_state1; F.hs2 = host_state2; F.ha1 = host_absmax1; F.ha2 = host_absmax2;
            F.n = n;
            F.dirty = false;
            F.wb_pending = false;            // the copy-in followed every write-back (tail)
            pool->where[{host_state1, i}] = f;
            ++pool->page_ins;
        }
        if (e != hipSuccess) break;
        PoolFrame& F = pool->fr[(size_t)f];
        uint8_t* buf = pool->frames + (int64_t)f * pool->L.bytes;
        if (int rc = run_step(hp, step, static_cast<uint8_t*>(p) + c0 * es, static_cast<const uint8_t*>(g) + c0 * es,
                              dtype, len, buf + pool->L.s1, two ? buf + pool->L.s2 : nullptr,
                              reinterpret_cast<float*>(buf + pool->L.a1),
                              two ? reinterpret_cast<float*>(buf + pool->L.a2) : nullptr, qmap1,
                              two ? qmap2 : nullptr, true, stream, fn))
            return rc;
        chk(hipEventRecord(F.comp, sc));
        F.stepped = true;
        F.last_stream = sc;
        F.dirty = true;
        F.tick = ++pool->tick;
    }
    return device_status(e, fn);
}

int bitopt_page_pool_flush(bitopt_page_pool* pool, int32_t evict, void* stream) {
    const char* fn = "bitopt_page_pool_flush";
    if (!pool) return fail(BITOPT_ERR_INVALID_ARG, "%s: pool is NULL", fn);
    if (int rc = pool_device_ok(pool, fn)) return rc;
    hipStream_t sc = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    bool any = false;
    for (PoolFrame& F : pool->fr) {
        if (!F.key || !F.dirty) continue;
        if (!any) {
            chk(hipEventRecord(pool->start, sc));
            chk(hipStreamWaitEvent(pool->d2h, pool->start, 0));
            any = true;
        }
        chk(pool_write_back(pool, F, sc));
    }
    if (any) {
        chk(hipEventRecord(pool->tail, pool->d2h));
        ++pool->tail_seq;
    }
    // `stream` completes only after every write-back enqueued so far
    if (pool->tail_seq) chk(hipStreamWaitEvent(sc, pool->tail, 0));
    if (evict) {
        for (PoolFrame& F : pool->fr) {
            // a later copy-in into this frame waits for `tail`, which follows its last step
            F.key = nullptr;
            F.dirty = false;
        }
        pool->where.clear();
    }
    return device_status(e, fn);
}

int bitopt_page_pool_stats(const bitopt_page_pool* pool, int64_t* out4) {
    if (!pool || !out4) return fail(BITOPT_ERR_INVALID_ARG, "bitopt_page_pool_stats: NULL pointer");
    out4[0] = (int64_t)pool->where.size();
    out4[1] = pool->page_ins;
    out4[2] = pool->write_backs;
    out4[3] = pool->hits;
    return ok();
}

}  // extern "C"


namespace {

// Checks and launches of the tensor-wide step; ws: its workspace (device, 4-byte
// aligned, at least tensorwise_workspace_words() words), or NULL for the library's
// own scratch array.
int run_tensorwise(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype, int64_t n,
                   uint8_t* state1, uint8_t* state2, float* absmax1, float* absmax2, const float* qmap1,
                   const float* qmap2, void* workspace, bool own_scratch, void* stream, const char* fn) {
    if (!hp) return fail(BITOPT_ERR_INVALID_ARG, "%s: hp is NULL", fn);
    if (hp->blocksize != 0)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: blocksize must be 0 (one block for the tensor), got %d", fn,
                    hp->blocksize);
    bitopt_hparams h = *hp;
    h.blocksize = 256;                         // the shared checks know block sizes only
    if (int rc = check_hparams(&h, step, n, fn)) return rc;
    if (!valid_dtype(dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    if (n == 0) return ok();
    if (!p || !g || !state1 || !absmax1 || !qmap1 || (!own_scratch && !workspace) ||
        (two && (!state2 || !absmax2 || !qmap2)))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    if (own_scratch) {
        if (bitopt::tensorwise_workspace_words() > bitopt::tensorwise_scratch_words())
            return fail(BITOPT_ERR_UNSUPPORTED, "%s: the step needs %d workspace words, the scratch array holds %d",
                        fn, bitopt::tensorwise_workspace_words(), bitopt::tensorwise_scratch_words());
        hipError_t e = bitopt::tensorwise_scratch(&ws);
        if (e != hipSuccess) return device_status(e, fn);
    } else if (!aligned(workspace, 4)) {
        return fail(BITOPT_ERR_INVALID_ARG, "%s: workspace not 4-byte aligned", fn);
    }
    bitopt::StepArgs a{};
    a.p = p; a.g = g; a.s1 = state1; a.s2 = two ? state2 : nullptr; a.a1 = absmax1; a.a2 = two ? absmax2 : nullptr;
    a.q1 = qmap1; a.q2 = two ? qmap2 : qmap1;
    a.n = n;
    a.nb = 1;
    a.s = make_scalars(h, step);
    a.vec = vec_ok(&h, p, g, dtype, n, state1, two ? state2 : nullptr) ? 1 : 0;
    a.ws = ws;
    hipError_t e = bitopt::launch_tensorwise(a, hp->optimizer, dtype, hp->skip_zeros != 0,
                                             reinterpret_cast<hipStream_t>(stream));
    return device_status(e, fn);
}

}  // namespace

extern "C" {

int bitopt_step_8bit_tensorwise(const bitopt_hparams* hp, int32_t step, void* p, const void* g, int32_t dtype,
                                int64_t n, uint8_t* state1, uint8_t* state2, float* absmax1, float* absmax2,
                                const float* qmap1, const float* qmap2, void* workspace, void* stream) {
    return run_tensorwise(hp, step, p, g, dtype, n, state1, state2, absmax1, absmax2, qmap1, qmap2, workspace,
                          false, stream, "bitopt_step_8bit_tensorwise");
}

int bitopt_step_8bit_tensorwise_noalloc(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                        int32_t dtype, int64_t n, uint8_t* state1, uint8_t* state2,
                                        float* absmax1, float* absmax2, const float* qmap1, const float* qmap2,
                                        void* stream) {
    return run_tensorwise(hp, step, p, g, dtype, n, state1, state2, absmax1, absmax2, qmap1, qmap2, nullptr,
                          true, stream, "bitopt_step_8bit_tensorwise_noalloc");
}

int64_t bitopt_tensorwise_scratch_bytes(void) { return (int64_t)bitopt::tensorwise_scratch_words() * 4; }

int64_t bitopt_multi_workspace_bytes(int32_t count) {
    if (count < 0) return -1;
    return (int64_t)count * (int64_t)sizeof(bitopt::TensorDesc);
}

int bitopt_multi_plan_build(const bitopt_hparams* hp, const bitopt_tensor* tensors, int32_t count,
                            void* workspace, int64_t workspace_bytes, bitopt_multi_plan* plan, void* stream) {
    const char* fn = "bitopt_multi_plan_build";
    if (!plan) return fail(BITOPT_ERR_INVALID_ARG, "%s: plan is NULL", fn);
    std::memset(plan, 0, sizeof *plan);
    if (int rc = check_hparams(hp, 1, 0, fn)) return rc;
    if (count < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: count < 0", fn);
    if (count > 0 && !tensors) return fail(BITOPT_ERR_INVALID_ARG, "%s: tensors is NULL", fn);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    for (int32_t i = 0; i < count; ++i) {
        const bitopt_tensor& t = tensors[i];
        if (t.n < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: tensor %d: n < 0", fn, i);
        if (!valid_dtype(t.dtype)) return fail(BITOPT_ERR_INVALID_ARG, "%s: tensor %d: unknown dtype %d", fn, i, t.dtype);
        if (t.n == 0) continue;
        if (!t.p || !t.g || !t.state1 || (two && !t.state2))
            return fail(BITOPT_ERR_INVALID_ARG, "%s: tensor %d: NULL pointer", fn, i);
        if (t.is_8bit && (!t.absmax1 || (two && !t.absmax2)))
            return fail(BITOPT_ERR_INVALID_ARG, "%s: tensor %d: NULL absmax", fn, i);
    }
    if (count > 0 && (!workspace || workspace_bytes < bitopt_multi_workspace_bytes(count) || !aligned(workspace, 16)))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: workspace missing, too small or not 16-byte aligned", fn);

    // Group by kind (is_8bit, dtype), keeping call order inside a group; chunks of
    // at most kMaxTableTensors tensors and kMaxLaunchTiles tiles form one launch each.
    const int64_t te = tile_elems(hp->blocksize);
    std::vector<bitopt::TensorDesc> table;
    table.reserve((size_t)count);
    bitopt_multi_plan P{};
    P.optimizer = hp->optimizer;
    P.blocksize = hp->blocksize;
    P.workspace = workspace;
    auto push = [&](const bitopt_multi_launch& L) -> bool {
        if (P.nlaunch == BITOPT_MULTI_MAX_LAUNCHES) return false;
        P.launch[P.nlaunch++] = L;
        return true;
    };
    for (int kind8 = 1; kind8 >= 0; --kind8) {
        for (int dt = BITOPT_F32; dt <= BITOPT_BF16; ++dt) {
            bitopt_multi_launch L{kind8, dt, (int32_t)table.size(), 0, 0};
            for (int32_t i = 0; i < count; ++i) {
                const bitopt_tensor& t = tensors[i];
                if (t.n == 0 || (t.is_8bit != 0) != (kind8 != 0) || t.dtype != dt) continue;
                const int64_t tiles_t = (t.n + te - 1) / te;
                if (tiles_t > bitopt::kMaxLaunchTiles)
                    return fail(BITOPT_ERR_UNSUPPORTED, "%s: tensor %d: more than 2^32 - 1 tiles", fn, i);
                if (L.count == bitopt::kMaxTableTensors || L.tiles + tiles_t > bitopt::kMaxLaunchTiles) {
                    if (!push(L)) return fail(BITOPT_ERR_UNSUPPORTED, "%s: more than %d launches", fn, BITOPT_MULTI_MAX_LAUNCHES);
                    L = bitopt_multi_launch{kind8, dt, (int32_t)table.size(), 0, 0};
                }
                bitopt::TensorDesc d{};
                d.p = t.p; d.g = t.g; d.s1 = t.state1; d.s2 = two ? t.state2 : nullptr;
                d.a1 = kind8 ? t.absmax1 : nullptr; d.a2 = (kind8 && two) ? t.absmax2 : nullptr;
                d.n = t.n; d.nb = (t.n + hp->blocksize - 1) / hp->blocksize;
                d.tile0 = L.tiles;
                d.vec = vec_ok(hp, t.p, t.g, t.dtype, t.n, t.state1, two ? t.state2 : nullptr) ? 1 : 0;
                L.tiles += tiles_t;
                ++L.count;
                table.push_back(d);
            }
            if (L.count && !push(L)) return fail(BITOPT_ERR_UNSUPPORTED, "%s: more than %d launches", fn, BITOPT_MULTI_MAX_LAUNCHES);
        }
    }
    P.count = (int32_t)table.size();
    if (!table.empty()) {
        // The table is copied once, here; the host vector must outlive the copy, so the
        // call waits for the stream (planning is not part of a step).
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        hipError_t e = hipMemcpyAsync(workspace, table.data(), table.size() * sizeof(bitopt::TensorDesc),
                                      hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return device_status(e, fn);
    }
    *plan = P;
    return ok();
}

}  // extern "C"

namespace {

// The launches of a planned step; sdev: device scalars (or NULL: sc by value).
int run_planned(const bitopt_multi_plan* plan, const bitopt_hparams* hp, const bitopt::StepScalars& sc,
                const void* sdev, const float* qmap1, const float* qmap2, void* stream, const char* fn) {
    if (!plan) return fail(BITOPT_ERR_INVALID_ARG, "%s: plan is NULL", fn);
    if (hp->optimizer != plan->optimizer || hp->blocksize != plan->blocksize)
        return fail(BITOPT_ERR_INVALID_ARG, "%s: the plan was built for optimizer %d, blocksize %d", fn,
                    plan->optimizer, plan->blocksize);
    if (plan->nlaunch < 0 || plan->nlaunch > BITOPT_MULTI_MAX_LAUNCHES || (plan->nlaunch > 0 && !plan->workspace))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: not a plan made by bitopt_multi_plan_build", fn);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    bool any8 = false;
    for (int32_t i = 0; i < plan->nlaunch; ++i) any8 = any8 || plan->launch[i].kind8;
    if (any8 && (!qmap1 || (two && !qmap2))) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL qmap", fn);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < plan->nlaunch; ++i) {
        const bitopt_multi_launch& L = plan->launch[i];
        bitopt::StepArgs a{};
        a.q1 = qmap1; a.q2 = qmap2; a.s = sc;
        a.sdev = static_cast<const bitopt::StepScalars*>(sdev);
        a.table = reinterpret_cast<const bitopt::TensorDesc*>(plan->workspace) + L.first;
        a.ntab = L.count;
        a.total_tiles = L.tiles;
        a.n = 0; a.nb = 0; a.vec = 0;
        hipError_t e = dispatch_step(a, hp->optimizer, L.dtype, hp->blocksize, L.kind8 != 0, hp->skip_zeros != 0,
                                     hp->max_unorm > 0.0f, s);
        if (e != hipSuccess) return device_status(e, fn);
    }
    return ok();
}

}  // namespace

extern "C" {

int bitopt_step_multi_planned(const bitopt_multi_plan* plan, const bitopt_hparams* hp, int32_t step,
                              const float* qmap1, const float* qmap2, void* stream) {
    const char* fn = "bitopt_step_multi_planned";
    if (int rc = check_hparams(hp, step, 0, fn)) return rc;
    return run_planned(plan, hp, make_scalars(*hp, step), nullptr, qmap1, qmap2, stream, fn);
}

int64_t bitopt_device_scalars_bytes(void) { return (int64_t)sizeof(bitopt::StepScalars); }

int bitopt_device_scalars_write(const bitopt_hparams* hp, int32_t step, void* out, int64_t out_bytes) {
    const char* fn = "bitopt_device_scalars_write";
    if (int rc = check_hparams(hp, step, 0, fn)) return rc;
    if (!out) return fail(BITOPT_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (out_bytes < (int64_t)sizeof(bitopt::StepScalars))
        return fail(BITOPT_ERR_INVALID_ARG, "%s: out holds %lld bytes, %lld needed", fn, (long long)out_bytes,
                    (long long)sizeof(bitopt::StepScalars));
    const bitopt::StepScalars sc = make_scalars(*hp, step);
    std::memcpy(out, &sc, sizeof sc);
    return ok();
}

int bitopt_step_multi_planned_dscalars(const bitopt_multi_plan* plan, const bitopt_hparams* hp, const void* scalars,
                                       const float* qmap1, const float* qmap2, void* stream) {
    const char* fn = "bitopt_step_multi_planned_dscalars";
    if (int rc = check_hparams(hp, 1, 0, fn)) return rc;
    if (!scalars) return fail(BITOPT_ERR_INVALID_ARG, "%s: scalars is NULL", fn);
    if (!aligned(scalars, 16)) return fail(BITOPT_ERR_INVALID_ARG, "%s: scalars not 16-byte aligned", fn);
    return run_planned(plan, hp, bitopt::StepScalars{}, scalars, qmap1, qmap2, stream, fn);
}

int bitopt_step_multi(const bitopt_hparams* hp, int32_t step, const bitopt_tensor* tensors, int32_t count,
                      const float* qmap1, const float* qmap2, void* workspace, int64_t workspace_bytes,
                      void* stream) {
    const char* fn = "bitopt_step_multi";
    if (int rc = check_hparams(hp, step, 0, fn)) return rc;
    if (count < 0) return fail(BITOPT_ERR_INVALID_ARG, "%s: count < 0", fn);
    if (count == 0) return ok();
    if (!tensors) return fail(BITOPT_ERR_INVALID_ARG, "%s: tensors is NULL", fn);
    const bool two = hp->optimizer == BITOPT_ADAM || hp->optimizer == BITOPT_ADEMAMIX;
    bool any8 = false;
    for (int32_t i = 0; i < count; ++i) any8 = any8 || (tensors[i].is_8bit && tensors[i].n > 0);
    if (any8 && (!qmap1 || (two && !qmap2))) return fail(BITOPT_ERR_INVALID_ARG, "%s: NULL qmap", fn);
    bitopt_multi_plan plan;
    if (int rc = bitopt_multi_plan_build(hp, tensors, count, workspace, workspace_bytes, &plan, stream)) return rc;
    return bitopt_step_multi_planned(&plan, hp, step, qmap1, qmap2, stream);
}

}  // extern "C"
