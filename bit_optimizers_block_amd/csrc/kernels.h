// kernels.h -- gfx950 device code of libbitopt: the fused 8-bit block-wise
// optimizer step, its 32-bit (identity codec) twin and the block-wise codec.
//
// Work decomposition (CDNA4, wave64).  A wavefront owns a tile of NQ quads; quad q
// of lane l holds elements q*256 + 4l .. +3, so every load/store instruction of the
// wave covers one contiguous 256-element span (16 B/lane for fp32, 8 B/lane for
// 16-bit, 4 B/lane of codes) and carries the non-temporal hint.  Blocks of 256 are
// single quads (four per tile): their absmax comes from one reduce-scatter across
// the wave; a block of 2048 is a whole tile, reduced by DPP row shifts, row
// broadcasts and readlane.  Full tiles keep the whole tile in registers and read
// each input once; a ragged last tile (or any tile of a misaligned tensor) takes a
// two-pass path that holds one quad at a time.  The 256-entry codebooks sit in
// LDS; decoding is one LDS gather.  Encoding with a standard dynamic map is one
// bucket lookup (exponent and top mantissa bits of x) plus one comparison with an
// fp32 decision threshold, both in LDS; any other map falls back to a branch-free
// binary search plus one neighbour comparison.  Both give the nearest entry (fp32
// distance, ties to the lower index).
//
// Arithmetic.  Each element operation is one IEEE fp32 operation in a fixed order
// (the build disables FMA contraction and keeps correctly rounded division and
// square root), so results do not depend on the tiling and are reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bitopt_tables.h"   // generated: constant search tables of the standard maps
#include "search_layout.h"

namespace bitopt {

constexpr int kF32 = 0, kF16 = 1, kBF16 = 2;
constexpr int kAdam = 0, kAdemamix = 1, kMomentum = 2, kLion = 3, kRmsprop = 4, kAdagrad = 5;
constexpr int kThreads = 256;              // 4 waves per workgroup
constexpr int kWavesPerGroup = kThreads / 64;

// Per-step scalars, formed on the host in double and rounded once to fp32.
struct StepScalars {
    float lr, b1, b2, eps, wd;
    float omb1, omb2, ic1, rs2, decay;
    float b3t, omb3, alpha_t;
    float max_unorm;
    float lric1;         // fl(lr * ic1): the Adam step's numerator scale in the estimate path
    int32_t fast_root;   // eps <= 2^60, rs2 <= 2^20, lric1 zero or normal (see root_delta_estimate)
};

// One tensor of a multi-tensor launch (device table entry): the same fields as a
// single-tensor call plus the index of its first tile in the launch.
struct TensorDesc {
    void* p;
    const void* g;
    void* s1;
    void* s2;
    float* a1;
    float* a2;
    int64_t n;
    int64_t nb;
    int64_t tile0;
    int32_t vec;
    int32_t pad;
};
constexpr int kMaxTableTensors = 1024;     // tensors per multi-tensor launch
constexpr int64_t kMaxLaunchTiles = 0xFFFFFFFFll;   // tiles per multi-tensor launch (uint32 first-tile indices)

struct StepArgs {
    void* p;
    const void* g;
    void* s1;          // 8-bit: uint8 codes; 32-bit: fp32 states.  AdEMAMix: m1 then m2.
    void* s2;
    float* a1;         // absmax (8-bit only).  AdEMAMix: m1's nb then m2's nb.
    float* a2;
    const float* q1;   // signed map
    const float* q2;   // unsigned map
    int64_t n;
    int64_t nb;        // number of blocks
    int32_t vec;       // 1: every buffer is aligned for the vector path
    StepScalars s;
    const TensorDesc* table;   // multi-tensor launch: ntab tensors (the fields above unused)
    int32_t ntab;
    int64_t total_tiles;
    uint32_t* ws;              // tensor-wide step: workspace shared by its passes
    int32_t parts;             // tensor-wide step: groups of pass 1 (partial results in ws)
    const StepScalars* sdev;   // multi-tensor launch: scalars read from device memory (else s)
};

template <int OPT> struct NumStates { static constexpr int v = OPT == kAdemamix ? 3 : (OPT == kAdam ? 2 : 1); };
// 1-state optimizers whose state is never negative: their map is expected to be the unsigned one.
template <int OPT> struct UnsignedState1 { static constexpr int v = (OPT == kRmsprop || OPT == kAdagrad) ? 1 : 0; };

// ---------------------------------------------------------------- number formats

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streamed arrays (parameters, gradients, codes, fp32 states) are touched once per
// step: their loads and stores carry the non-temporal hint so they do not displace
// reusable lines in the caches.
#ifndef BITOPT_NONTEMPORAL
#define BITOPT_NONTEMPORAL 1
#endif

// Every tensor the kernels touch lives in device (global) memory.  Pointers read from
// the multi-tensor descriptor table would otherwise be generic, and generic (flat)
// accesses share the LDS wait counter, so each LDS wait would also wait for every
// outstanding HBM load.  Accesses go through gbl() so they compile to global ones.
#define BITOPT_GLOBAL __attribute__((address_space(1)))
template <class T> __device__ __forceinline__ BITOPT_GLOBAL T* gbl(T* p) { return (BITOPT_GLOBAL T*)p; }

template <class T> __device__ __forceinline__ T ld_stream(const T* p) {
    if constexpr (BITOPT_NONTEMPORAL) return __builtin_nontemporal_load(gbl(p));
    else return *gbl(p);
}
template <class T> __device__ __forceinline__ void st_stream(T v, T* p) {
    if constexpr (BITOPT_NONTEMPORAL) __builtin_nontemporal_store(v, gbl(p));
    else *gbl(p) = v;
}

template <int DT> struct Elem;
template <> struct Elem<kF32>  { using T = float;    using Raw4 = u32x4; };
template <> struct Elem<kF16>  { using T = uint16_t; using Raw4 = u32x2; };
template <> struct Elem<kBF16> { using T = uint16_t; using Raw4 = u32x2; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
// fp32 -> fp16 / bf16, round to nearest even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values packed into one 32-bit word (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <int DT> __device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (DT == kF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int DT> __device__ __forceinline__ float widen(uint32_t bits) {
    if constexpr (DT == kF32) return __uint_as_float(bits);
    else if constexpr (DT == kF16) return half_bits_to_f32(bits & 0xffffu);
    else return bf16_bits_to_f32(bits & 0xffffu);
}
template <int DT> __device__ __forceinline__ uint32_t narrow(float f) {
    if constexpr (DT == kF32) return __float_as_uint(f);
    else if constexpr (DT == kF16) return f32_to_half_bits(f);
    else return f32_to_bf16_bits(f);
}

// Four consecutive elements starting at element index e (vector path: aligned).
template <int DT> __device__ __forceinline__ void load4(const void* base, int64_t e, float v[4]) {
    using Raw4 = typename Elem<DT>::Raw4;
    const Raw4 r = ld_stream(reinterpret_cast<const Raw4*>(reinterpret_cast<const typename Elem<DT>::T*>(base) + e));
    if constexpr (DT == kF32) {
        v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
        v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
    } else {
        v[0] = widen<DT>(r.x); v[1] = widen<DT>(r.x >> 16);
        v[2] = widen<DT>(r.y); v[3] = widen<DT>(r.y >> 16);
    }
}
template <int DT> __device__ __forceinline__ void store4(void* base, int64_t e, const float v[4]) {
    using Raw4 = typename Elem<DT>::Raw4;
    Raw4 r;
    if constexpr (DT == kF32) {
        r.x = __float_as_uint(v[0]); r.y = __float_as_uint(v[1]);
        r.z = __float_as_uint(v[2]); r.w = __float_as_uint(v[3]);
    } else {
        r.x = narrow2<DT>(v[0], v[1]);
        r.y = narrow2<DT>(v[2], v[3]);
    }
    st_stream(r, reinterpret_cast<Raw4*>(reinterpret_cast<typename Elem<DT>::T*>(base) + e));
}
// Guarded element access (tail tiles and unaligned buffers).
template <int DT> __device__ __forceinline__ float load1(const void* base, int64_t e) {
    const typename Elem<DT>::T x = gbl(reinterpret_cast<const typename Elem<DT>::T*>(base))[e];
    if constexpr (DT == kF32) return x;
    else return widen<DT>((uint32_t)x);
}
template <int DT> __device__ __forceinline__ void store1(void* base, int64_t e, float v) {
    if constexpr (DT == kF32) gbl(reinterpret_cast<float*>(base))[e] = v;
    else gbl(reinterpret_cast<uint16_t*>(base))[e] = (uint16_t)narrow<DT>(v);
}

// ---------------------------------------------------------------- wave reductions

// Maxima of non-negative floats are taken on their bit patterns as integers (the
// same order), which avoids the NaN-quieting moves a float max needs on values that
// arrive through lane exchanges.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_or_zero(int v) {
    // Lanes whose source lane is outside the pattern, or whose row is masked off,
    // read 0 (the identity of a max over non-negative values).
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Max over the 64 lanes of non-negative values; the result is wave-uniform.
// row_shr 1,2,4,8 leave each row's max in its lane 15; row_bcast15 and row_bcast31
// carry it across rows into lane 63, which is then read as a scalar.
__device__ __forceinline__ float wave_max_nonneg(float f) {
    int v = __float_as_int(f);
    v = max(v, dpp_or_zero<0x111, 0xF>(v));
    v = max(v, dpp_or_zero<0x112, 0xF>(v));
    v = max(v, dpp_or_zero<0x114, 0xF>(v));
    v = max(v, dpp_or_zero<0x118, 0xF>(v));
    v = max(v, dpp_or_zero<0x142, 0xA>(v));
    v = max(v, dpp_or_zero<0x143, 0xC>(v));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ bool wave_any(bool pred) { return __ballot(pred) != 0ull; }

// Butterfly sum: every lane adds the same pair at each level, so all lanes end with
// bit-identical totals.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Max over the 16 lanes of each DPP row (every lane ends with its row's max).
template <int CTRL>
__device__ __forceinline__ int dpp_rot(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ int row_max_nonneg(int v) {
    v = max(v, dpp_rot<0x128>(v));    // row_ror 8, 4, 2, 1
    v = max(v, dpp_rot<0x124>(v));
    v = max(v, dpp_rot<0x122>(v));
    v = max(v, dpp_rot<0x121>(v));
    return v;
}

// ---------------------------------------------------------------- codebook search

// Nearest entry of a sorted 256-entry map Q (in LDS) to x: the largest i in
// [0, 254] with Q[i] <= x (or 0), then i+1 if it is strictly closer in fp32.  A NaN
// value (from a non-finite state) is encoded as +0 is, as the table encoder does.
__device__ __forceinline__ uint32_t nearest_code(const float* Q, float x) {
    x = (x == x) ? x : 0.0f;
    int pos = 0;
#pragma unroll
    for (int s = 128; s >= 1; s >>= 1) pos = (Q[pos + s] <= x) ? pos + s : pos;
    const int i = pos > 254 ? 254 : pos;
    const float lo = Q[i], hi = Q[i + 1];
    const float du = hi - x;
    const float dd = x - lo;
    return du < dd ? (uint32_t)(i + 1) : (uint32_t)i;
}

// A codebook staged in LDS: the map itself, and for the standard maps the
// decision thresholds tau and the bucket table (see gen_tables.cpp).
struct MapLDS {
    const float* Q;
    const float* tau;
    const uint8_t* bkt;
};

// Nearest code.  FAST (standard maps): x is the normalized value scaled by
// 2^-kShift (see search_layout.h), and one bucket lookup plus one threshold
// comparison give code = bkt[idx(x)] + (x >= tau'[bkt[idx(x)]]), equal to the
// nearest-entry rule for every finite value.  NONNEG: the value is known to be
// non-negative (a second-moment state), so the sign term of the index is dropped.
// Otherwise x is the plain normalized value and the binary search above applies.
template <bool FAST, bool NONNEG = false>
__device__ __forceinline__ uint32_t encode(const MapLDS& m, float x) {
    if constexpr (FAST) {
        using namespace search;
        const uint32_t bits = __float_as_uint(x);
        const uint32_t key = (bits >> 16) & (uint32_t)(kNBH - 1);
        const uint32_t idx = (uint32_t)kNBH + (NONNEG ? key : (key ^ (uint32_t)((int32_t)bits >> 31)));
        const uint32_t c = m.bkt[idx];
        return c + (x >= m.tau[c] ? 1u : 0u);
    } else {
        return nearest_code(m.Q, x);
    }
}

// The table encoder on the four values of a quad, packed into one code word (value i
// in byte i).  The four bucket reads are issued together, then the four threshold
// reads, so the wave waits for LDS twice per quad rather than twice per element.
#ifndef BITOPT_ENCODE_GROUPS
#define BITOPT_ENCODE_GROUPS 1
#endif
template <bool NONNEG>
__device__ __forceinline__ uint32_t encode_quad(const MapLDS& m, const float (&y)[4]) {
    using namespace search;
    uint32_t c[4];
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t bits = __float_as_uint(y[i]);
        const uint32_t key = (bits >> 16) & (uint32_t)(kNBH - 1);
        const uint32_t idx = (uint32_t)kNBH + (NONNEG ? key : (key ^ (uint32_t)((int32_t)bits >> 31)));
        c[i] = m.bkt[idx];
    }
    if constexpr (BITOPT_ENCODE_GROUPS) {
        __builtin_amdgcn_sched_group_barrier(0x002, NONNEG ? 4 : 12, 0);   // bucket indices
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                  // bucket reads
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = m.tau[c[i]];
    if constexpr (BITOPT_ENCODE_GROUPS) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                  // threshold addresses
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                  // threshold reads
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) x |= (c[i] + (y[i] >= t[i] ? 1u : 0u)) << (8 * i);
    return x;
}

// The table encoder's scale, folded into a block's reciprocal r: r * 2^-kShift.  It
// gives the scaled value exactly when r >= 2^(kShift - 126) or r == 0; a block with a
// smaller reciprocal (absmax above 2^30) takes the binary search instead.
constexpr float kEncScale = 0x1p-96f;
static_assert(search::kShift == 96 && search::kMinRecipExp == -30, "encoder scale");
__device__ __forceinline__ bool table_recip_ok(float r) { return r >= 0x1p-30f || r == 0.0f; }

// Stage up to two codebooks into LDS.  Map 1 is expected to be the standard signed
// map (EXP1 = 1: the unsigned one) and map 2 the standard unsigned one, so their
// search tables are fetched
// together with the maps (one round of loads, one barrier).  Each wave votes on
// which standard map each staged map equals; if the group's vote shows the
// standard maps in the other assignment, the tables are staged again.  Returns
// whether the table encoder applies (uniform over the group); otherwise the
// caller uses the binary search over the staged maps.
template <int NMAPS, int EXP1 = 0>
__device__ __forceinline__ bool stage_maps(const float* q1, const float* q2, float* Q1, float* Q2,
                                           float* T1, float* T2, uint8_t* B1, uint8_t* B2, uint32_t* vote) {
    constexpr int NV = search::kNB / 16;                 // 16-byte words per bucket table
    static_assert(search::kNB % 16 == 0 && NV <= 2 * kThreads, "bucket table staging");
    const int tid = threadIdx.x;
    const u32x4* bs = reinterpret_cast<const u32x4*>(kStdBucket0);
    const u32x4* bu = reinterpret_cast<const u32x4*>(kStdBucket1);
    const bool two = tid + kThreads < NV;
    // every load first
    const uint32_t v1 = __float_as_uint(gbl(q1)[tid]);
    const uint32_t v2 = NMAPS > 1 ? __float_as_uint(gbl(q2)[tid]) : 0u;
    const uint32_t s0 = kStdQ0[tid], s1 = kStdQ1[tid];
    const uint32_t t1 = EXP1 ? kStdTau1[tid] : kStdTau0[tid];
    const uint32_t t2 = NMAPS > 1 ? kStdTau1[tid] : 0u;
    const u32x4* b1src = EXP1 ? bu : bs;
    const u32x4 b1a = b1src[tid];
    const u32x4 b1b = two ? b1src[tid + kThreads] : u32x4{0u, 0u, 0u, 0u};
    u32x4 b2a = {0u, 0u, 0u, 0u}, b2b = {0u, 0u, 0u, 0u};
    if constexpr (NMAPS > 1) {
        b2a = bu[tid];
        if (two) b2b = bu[tid + kThreads];
    }
    Q1[tid] = __uint_as_float(v1);
    T1[tid] = __uint_as_float(t1);
    reinterpret_cast<u32x4*>(B1)[tid] = b1a;
    if (two) reinterpret_cast<u32x4*>(B1)[tid + kThreads] = b1b;
    if constexpr (NMAPS > 1) {
        Q2[tid] = __uint_as_float(v2);
        T2[tid] = __uint_as_float(t2);
        reinterpret_cast<u32x4*>(B2)[tid] = b2a;
        if (two) reinterpret_cast<u32x4*>(B2)[tid + kThreads] = b2b;
    }
    // bit 0/1: map 1 equals the standard signed/unsigned map; bits 2/3: the same for map 2
    uint32_t bits = 0;
    if (__ballot(v1 != s0) == 0ull) bits |= 1u;
    if (__ballot(v1 != s1) == 0ull) bits |= 2u;
    if constexpr (NMAPS > 1) {
        if (__ballot(v2 != s0) == 0ull) bits |= 4u;
        if (__ballot(v2 != s1) == 0ull) bits |= 8u;
    }
    if ((tid & 63) == 0) vote[tid >> 6] = bits;
    __syncthreads();
    uint32_t all = vote[0];
#pragma unroll
    for (int w = 1; w < kWavesPerGroup; ++w) all &= vote[w];
    if ((all & (EXP1 ? 2u : 1u)) && (NMAPS == 1 || (all & 8u))) return true;
    const int w1 = (all & 1u) ? 0 : (all & 2u) ? 1 : -1;
    const int w2 = NMAPS == 1 ? 0 : (all & 4u) ? 0 : (all & 8u) ? 1 : -1;
    if (w1 < 0 || w2 < 0) return false;
    // standard maps in the other assignment (nothing has read the tables yet)
    const int which[2] = {w1, w2};
    float* T[2] = {T1, T2};
    uint8_t* Bk[2] = {B1, B2};
#pragma unroll
    for (int k = 0; k < NMAPS; ++k) {
        const uint32_t* tsrc = which[k] ? kStdTau1 : kStdTau0;
        const u32x4* bsrc = which[k] ? bu : bs;
        T[k][tid] = __uint_as_float(tsrc[tid]);
        reinterpret_cast<u32x4*>(Bk[k])[tid] = bsrc[tid];
        if (two) reinterpret_cast<u32x4*>(Bk[k])[tid + kThreads] = bsrc[tid + kThreads];
    }
    __syncthreads();
    return true;
}

// ---------------------------------------------------------------- optimizer updates

// Correctly rounded square root for v == 0 and v >= 2^-96 (and +inf, NaN): the hardware
// estimate, within one ulp, is moved to a neighbour when the fused residual
// v - neighbour * estimate shows that neighbour is the rounded root.  This is the
// general correctly rounded expansion without its input scaling and its final
// zero/infinity select, and gives the same bits wherever that scaling is not
// applied; positive v below 2^-96 need the scaling (see quad_needs_scaling).
__device__ __forceinline__ float sqrt_rn_unscaled(float v) {
    const float s = __builtin_amdgcn_sqrtf(v);
    const float dn = __uint_as_float(__float_as_uint(s) - 1u);
    const float up = __uint_as_float(__float_as_uint(s) + 1u);
    const float rdn = __builtin_fmaf(-dn, s, v);
    const float rup = __builtin_fmaf(-up, s, v);
    const float r = rdn <= 0.0f ? dn : s;
    return rup > 0.0f ? up : r;
}
// Whether any of four non-negative values lies in (0, 2^-96), i.e. has bits in
// 1 .. 0x0F7FFFFF: one unsigned minimum of the bit patterns minus one (0 wraps high).
__device__ __forceinline__ bool quad_needs_scaling(const float (&v)[4]) {
    const uint32_t m01 = min(__float_as_uint(v[0]) - 1u, __float_as_uint(v[1]) - 1u);
    const uint32_t m23 = min(__float_as_uint(v[2]) - 1u, __float_as_uint(v[3]) - 1u);
    return min(m01, m23) < 0x0F7FFFFFu;
}

// Optimizers whose step divides by a root of a second-moment state.
template <int OPT> struct HasRoot {
    static constexpr bool v = OPT == kAdam || OPT == kAdemamix || OPT == kRmsprop || OPT == kAdagrad;
};
// Index of that state (v, nu, square_avg, sum) in the state vector.
template <int OPT> struct RootState { static constexpr int v = OPT == kAdemamix ? 2 : (OPT == kAdam ? 1 : 0); };

// Root optimizers: the new states (Adam {m, v}; AdEMAMix {m1, m2, nu}; RMSprop
// {square_avg}; Adagrad {sum}).  RMSprop and Adagrad fold the decay into the
// gradient, g' = g + wd * p.
template <int OPT>
__device__ __forceinline__ void moments(const StepScalars& s, float p, float g, float st[3]) {
    float t1, t2;
    if constexpr (OPT == kAdam) {
        t1 = s.b1 * st[0]; t2 = s.omb1 * g; st[0] = t1 + t2;
        const float gg = g * g;
        t1 = s.b2 * st[1]; t2 = s.omb2 * gg; st[1] = t1 + t2;
    } else if constexpr (OPT == kAdemamix) {
        t1 = s.b1 * st[0]; t2 = s.omb1 * g; st[0] = t1 + t2;
        t1 = s.b3t * st[1]; t2 = s.omb3 * g; st[1] = t1 + t2;
        const float gg = g * g;
        t1 = s.b2 * st[2]; t2 = s.omb2 * gg; st[2] = t1 + t2;
    } else if constexpr (OPT == kRmsprop) {
        t1 = s.wd * p;
        const float g2 = g + t1;
        const float gg = g2 * g2;
        t1 = s.b1 * st[0]; t2 = s.omb1 * gg; st[0] = t1 + t2;
    } else {
        static_assert(OPT == kAdagrad, "moments of a root optimizer");
        t1 = s.wd * p;
        const float g2 = g + t1;
        const float gg = g2 * g2;
        st[0] = st[0] + gg;
    }
}

// Root optimizers: the parameter step from the new states, d = lr * u with
//   Adam/AdEMAMix  u = (m * ic1 [+ alpha_t * m2]) / (sqrt(v) * rs2 + eps)
//   RMSprop/Adagrad  u = g' / (sqrt(state) + eps).
// UNSCALED: the caller has checked that no state needs the scaled square root.
template <int OPT, bool UNSCALED>
__device__ __forceinline__ float root_delta(const StepScalars& s, float p, float g, const float st[3]) {
    const float v = st[RootState<OPT>::v];
    const float r = UNSCALED ? sqrt_rn_unscaled(v) : sqrtf(v);
    float u;
    if constexpr (OPT == kAdam || OPT == kAdemamix) {
        float den = r * s.rs2;
        den = den + s.eps;
        float num = st[0] * s.ic1;
        if constexpr (OPT == kAdemamix) {
            const float t2 = s.alpha_t * st[1];
            num = num + t2;
        }
        u = num / den;
    } else {
        const float t1 = s.wd * p;
        const float g2 = g + t1;
        const float den = r + s.eps;
        u = g2 / den;
    }
    return s.lr * u;
}

// The same parameter step from the hardware estimates: square root and reciprocal
// each within one ulp (for v outside (0, 2^-96) and a denominator below 2^85, which
// eps <= 2^60 and rs2 <= 2^20 ensure).  The denominator is one fused multiply-add;
// Adam scales m once by fl(lr * ic1) (zero or normal) instead of by ic1 and then lr.
// Against root_delta's roundings this leaves the step within 14 units of 2^-24
// relative (Adam: 8 units from the exact quotient here, 6 there; AdEMAMix and the
// others fewer), plus 2^-140 absolute where it is subnormal.
template <int OPT>
__device__ __forceinline__ float root_delta_estimate(const StepScalars& s, float p, float g, const float st[3]) {
    const float r = __builtin_amdgcn_sqrtf(st[RootState<OPT>::v]);
    if constexpr (OPT == kAdam) {
        const float den = __builtin_fmaf(r, s.rs2, s.eps);
        const float num = st[0] * s.lric1;
        return num * __builtin_amdgcn_rcpf(den);
    }
    float num, den;
    if constexpr (OPT == kAdemamix) {
        den = __builtin_fmaf(r, s.rs2, s.eps);
        num = st[0] * s.ic1;
        const float t2 = s.alpha_t * st[1];
        num = num + t2;
    } else {
        const float t1 = s.wd * p;
        num = g + t1;
        den = r + s.eps;
    }
    const float u = num * __builtin_amdgcn_rcpf(den);
    return s.lr * u;
}

// New 16-bit parameters from estimated steps, two elements at a time, when the
// estimate provably gives the exact path's bits: with e = |d| 2^-19 + 2^-120 -- more
// than the distance of d from the exact step dx (14 * 2^-24 |d| + 2^-140) plus the
// rounding of d +- e, so that the rounded sums d + e and d - e still bracket dx --
// the bounds lo = fl(pd - (d + e)) and hi = fl(pd - (d - e)) enclose fl(pd - dx)
// (correctly rounded subtraction is monotone); when lo and hi round to the same
// 16-bit value, so does fl(pd - dx), the exact path's parameter.  w receives the two
// lo values rounded and packed; the result is whether both pairs of bounds round
// alike.  emax accumulates the margins' bit patterns (e >= 0, so they order as
// values, and NaN lies above +inf): the caller requires emax < +inf, which rejects a
// step that is NaN or infinite.
// The same test for one element, whose bounds are rounded in one pair: fl(pd - d) is
// then the result (the form that keeps the fewest values live).
template <int DT>
__device__ __forceinline__ bool rounds_alike(float pd, float d) {
    const float e = __builtin_fmaf(__builtin_fabsf(d), 0x1p-19f, 0x1p-120f);
    const float dhi = d + e;
    const float dlo = d - e;
    const uint32_t w = narrow2<DT>(pd - dhi, pd - dlo);
    return (w & 0xffffu) == (w >> 16) && e < __builtin_inff();
}

template <int DT>
__device__ __forceinline__ bool pair_rounds_alike(float pd0, float d0, float pd1, float d1, uint32_t& w,
                                                  uint32_t& emax) {
    const float e0 = __builtin_fmaf(__builtin_fabsf(d0), 0x1p-19f, 0x1p-120f);
    const float e1 = __builtin_fmaf(__builtin_fabsf(d1), 0x1p-19f, 0x1p-120f);
    const float dhi0 = d0 + e0, dlo0 = d0 - e0;
    const float dhi1 = d1 + e1, dlo1 = d1 - e1;
    emax = max(emax, max(__float_as_uint(e0), __float_as_uint(e1)));
    w = narrow2<DT>(pd0 - dhi0, pd1 - dhi1);
    return w == narrow2<DT>(pd0 - dlo0, pd1 - dlo1);
}

// One element of one step.  st[] holds the decoded states on entry and the new
// states on exit; the parameter step delta is returned through d.
// Adam/AdEMAMix: st = {m, v} / {m1, m2, nu};  Momentum: {buf};  Lion: {m};
// RMSprop: {square_avg};  Adagrad: {sum}.
template <int OPT>
__device__ __forceinline__ void update_elem(const StepScalars& s, float p, float g, float st[3], float& d) {
    float t1, t2;
    if constexpr (HasRoot<OPT>::v) {
        moments<OPT>(s, p, g, st);
        d = root_delta<OPT, false>(s, p, g, st);
    } else if constexpr (OPT == kMomentum) {
        float buf = st[0];
        t1 = s.wd * p;
        const float g2 = g + t1;
        t1 = s.b1 * buf; buf = t1 + g2;
        d = s.lr * buf;
        st[0] = buf;
    } else {   // Lion
        float m = st[0];
        t1 = s.b1 * m; t2 = s.omb1 * g;
        const float c = t1 + t2;
        const float sg = c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
        d = s.lr * sg;
        t1 = s.b2 * m; t2 = s.omb2 * g; m = t1 + t2;
        st[0] = m;
    }
}

// The parameter before the step is subtracted: p * (1 - lr*wd) for decoupled decay,
// p itself where the decay is folded into the gradient.
template <int OPT>
__device__ __forceinline__ float decayed(const StepScalars& s, float p) {
    if constexpr (OPT == kMomentum || OPT == kRmsprop || OPT == kAdagrad) return p;
    else return p * s.decay;
}

template <int OPT>
__device__ __forceinline__ float apply_step(const StepScalars& s, float p, float d) {
    const float pd = decayed<OPT>(s, p);
    return pd - d;
}

// Location of state k: AdEMAMix keeps m1 and m2 in slot 1 (m2 after n elements /
// nb blocks) and nu in slot 2; the others keep state 0 in slot 1, state 1 in slot 2.
template <int OPT> struct Slot {
    static __device__ __forceinline__ int which(int k) { return (OPT == kAdemamix) ? (k < 2 ? 0 : 1) : k; }
    static __device__ __forceinline__ int64_t elem_off(int k, int64_t n) { return (OPT == kAdemamix && k == 1) ? n : 0; }
    static __device__ __forceinline__ int64_t block_off(int k, int64_t nb) { return (OPT == kAdemamix && k == 1) ? nb : 0; }
};

// ---------------------------------------------------------------- tile layouts

// A wave tile is NQ quads: quad q of lane l holds elements q*256 + 4l .. +3, so every
// load and store instruction of the wave covers one contiguous 256-element span
// (1 KB of fp32, 256 B of codes) -- the pattern the memory system streams best.
// A block of BS elements is QPB = BS/256 consecutive quads; a tile holds BPT blocks.
template <int BS> struct Layout {
    static constexpr int NQ = BS >= 1024 ? BS / 256 : 4;
    static constexpr int TE = NQ * 256;
    static constexpr int QPB = BS / 256;
    static constexpr int BPT = NQ / QPB;
    static __device__ __forceinline__ int64_t elem(int64_t base, int lane, int q) { return base + q * 256 + lane * 4; }
};

// Block absmax and its reciprocal for the BPT blocks of a tile, from each lane's
// partial maxima m[b] (non-negative), left in lanes: with one block per tile every
// lane holds the pair; with four, row b (lanes 16b .. 16b+15) holds block b's.
// One block per tile: a wave max.  Four blocks per tile: a reduce-scatter -- two
// exchanges between lane halves and row pairs leave row r with the partial max of
// block r, a row reduction completes it, and one reciprocal serves all four blocks.
// Normalization of a block with absmax u: values x map to (x * c) * r with one
// correctly rounded reciprocal r = 1/(u * c) (r = 0 when u = 0).  c = 2^24 when u is
// subnormal, whose plain reciprocal can exceed the fp32 range; otherwise c = 1,
// i.e. the plain x * (1/u).  Both forms give the same bits wherever 1/u is finite.
__device__ __forceinline__ void block_recip(float u, float& r, float& c) {
    c = (u < 0x1p-126f) ? 0x1p24f : 1.0f;
    r = (u == 0.0f) ? 0.0f : 1.0f / (u * c);
}

template <int BPT>
__device__ __forceinline__ void block_absmax_lanes(const float (&m)[BPT], float& u, float& ru, float& cu) {
    if constexpr (BPT == 1) {
        u = wave_max_nonneg(m[0]);
    } else {
        static_assert(BPT == 4, "tiles hold one or four blocks");
        // gfx950 lane swaps: permlane32 exchanges the upper half of its first operand
        // with the lower half of its second, so after one swap and a max, lanes 0-31
        // hold block 0 (1) over both halves and lanes 32-63 block 2 (3); permlane16
        // then exchanges the odd rows of the first operand with the even rows of the
        // second, and a max leaves row r with the partial of block r over four lanes.
        int mi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) mi[b] = __float_as_int(m[b]);
        const auto s02 = __builtin_amdgcn_permlane32_swap(mi[0], mi[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(mi[1], mi[3], false, false);
        const int w02 = max((int)s02[0], (int)s02[1]);
        const int w13 = max((int)s13[0], (int)s13[1]);
        const auto r = __builtin_amdgcn_permlane16_swap(w02, w13, false, false);
        u = __int_as_float(row_max_nonneg(max((int)r[0], (int)r[1])));
    }
    block_recip(u, ru, cu);
}

// Whether the table encoder's scaled reciprocal r * 2^-kShift is exact: r >= 2^-30 or
// r == 0, on the bit pattern of a non-negative r (0 wraps to the top).
__device__ __forceinline__ bool recip_ok_bits(float r) {
    return __float_as_uint(r) - 1u >= __float_as_uint(0x1p-30f) - 1u;
}

// Block b's value of a pair left in lanes by block_absmax_lanes (wave-uniform).
template <int BPT>
__device__ __forceinline__ float block_value(float v, int b) {
    if constexpr (BPT == 1) return v;
    else return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), (64 / BPT) * b));
}

template <bool FULL>
__device__ __forceinline__ void store_code_word(uint8_t* cp, int64_t e, int64_t n, uint32_t w) {
    if constexpr (FULL) {
        st_stream(w, reinterpret_cast<uint32_t*>(cp + e));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e + i < n) gbl(cp)[e + i] = (uint8_t)(w >> (8 * i));
    }
}

// Encode the lane's values of one tile: per-block absmax, nearest codes of value *
// (1/absmax).  The new absmax is left in lanes (Al): with one block per tile in every
// lane, with four blocks in row b for block b.  Quads of blocks past the end hold
// zeros.  The table encoder serves every tile whose blocks have an absmax of at most
// 2^30 (a subnormal absmax with its 2^24 prescale: its scaled reciprocal stays
// normal); a larger absmax, or a map without tables, takes the binary search -- one
// element at a time, so that this path, which practical data never reaches, does not
// raise the kernel's register count.  The decisions are taken once per tile on the
// lanes' values (two ballots), and each quad reads its block's scaled reciprocal
// from the lane that holds it.
template <int BS, bool FAST, bool NONNEG, int NQ>
__device__ __forceinline__ void encode_tile(const MapLDS& M, const float (&v)[NQ][4], uint32_t w[NQ], float& Al) {
    using L = Layout<BS>;
    float m[L::BPT];
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) {
        float x = 0.0f;
#pragma unroll
        for (int qq = 0; qq < L::QPB; ++qq)
#pragma unroll
            for (int i = 0; i < 4; ++i) x = fmaxf(x, fabsf(v[b * L::QPB + qq][i]));
        m[b] = x;
    }
    float u, ru, cu;
    block_absmax_lanes<L::BPT>(m, u, ru, cu);
    Al = u;
    const bool table = FAST && !wave_any(!recip_ok_bits(ru));       // uniform
    const bool scaled = wave_any(cu != 1.0f);
    if (table) {
        const float rs = ru * kEncScale;
        auto tables = [&](auto prescale) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const float rq = block_value<L::BPT>(rs, q / L::QPB);
                const float cq = decltype(prescale)::value ? block_value<L::BPT>(cu, q / L::QPB) : 1.0f;
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = decltype(prescale)::value ? (v[q][i] * cq) * rq : v[q][i] * rq;
                w[q] = encode_quad<NONNEG>(M, y);
            }
        };
        if (!scaled) tables(std::false_type{});
        else tables(std::true_type{});
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float rq = block_value<L::BPT>(ru, q / L::QPB), cq = block_value<L::BPT>(cu, q / L::QPB);
            uint32_t x = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x |= encode<false>(M, (v[q][i] * cq) * rq) << (8 * i);
                __builtin_amdgcn_sched_barrier(0);
            }
            w[q] = x;
        }
    }
}

// encode_tile for a tile holding one block whose absmax u (uniform) is already known:
// a wave's half of a 2048-element block, the other half's maximum included.
template <int BS, bool FAST, bool NONNEG, int NQ>
__device__ __forceinline__ void encode_tile_given(const MapLDS& M, const float (&v)[NQ][4], uint32_t w[NQ],
                                                  float u) {
    static_assert(Layout<BS>::BPT == 1, "one block per tile");
    float ru, cu;
    block_recip(u, ru, cu);
    const bool table = FAST && recip_ok_bits(ru);       // uniform
    if (table) {
        const float rs = ru * kEncScale;
        const bool scaled = cu != 1.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = scaled ? (v[q][i] * cu) * rs : v[q][i] * rs;
            w[q] = encode_quad<NONNEG>(M, y);
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            uint32_t x = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x |= encode<false>(M, (v[q][i] * cu) * ru) << (8 * i);
                __builtin_amdgcn_sched_barrier(0);
            }
            w[q] = x;
        }
    }
}

// Store the new absmax of the tile's blocks from the lanes that hold them (see
// encode_tile); wmask: bit b set when block b is written (uniform).
template <int BPT>
__device__ __forceinline__ void store_absmax(float* am, int64_t blk0, int lane, float Al, uint32_t wmask) {
    if constexpr (BPT == 1) {
        if ((wmask & 1u) && lane == 0) gbl(am)[blk0] = Al;
    } else {
        const int b = lane >> 4;
        if ((lane & 15) == 0 && ((wmask >> b) & 1u)) gbl(am)[blk0 + b] = Al;
    }
}

// ---------------------------------------------------------------- fused step tile

// Raw inputs of one lane for one full tile, as loaded: parameter and gradient
// words, code words (8-bit) or fp32 states, and the tile's block absmax per state.
template <int DT, int OPT, int BS, bool QUANT>
struct TileRaw {
    static constexpr int NQ = Layout<BS>::NQ;
    static constexpr int BPT = Layout<BS>::BPT;
    static constexpr int NS = NumStates<OPT>::v;
    static constexpr int PW = DT == kF32 ? 4 : 2;           // 32-bit words per quad
    uint32_t p[NQ][PW], g[NQ][PW];
    uint32_t code[QUANT ? NS : 1][NQ];
    f32x4 fst[QUANT ? 1 : NS][NQ];
    float A[NS][BPT];
    uint32_t live;      // skip_zeros: bit b set when block b has a nonzero gradient (uniform)
};

// Whether a raw gradient word holds a nonzero value (-0 counts as zero): one fp32
// value, or two 16-bit ones.
template <int DT> __device__ __forceinline__ bool word_nonzero(uint32_t w) {
    if constexpr (DT == kF32) return (w & 0x7fffffffu) != 0u;
    else return (w & 0x7fff7fffu) != 0u;
}

template <int DT, int PW>
__device__ __forceinline__ void widen_words(const uint32_t (&w)[PW], float v[4]) {
    if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    } else {
        v[0] = widen<DT>(w[0]); v[1] = widen<DT>(w[0] >> 16);
        v[2] = widen<DT>(w[1]); v[3] = widen<DT>(w[1] >> 16);
    }
}

// A full tile: in range, every buffer aligned for the vector path.
template <int BS>
__device__ __forceinline__ bool tile_full(const StepArgs& a, int64_t t) {
    return a.vec && (t + 1) * Layout<BS>::TE <= a.n;
}

// The loads of one full tile (vector accesses), in two parts.  load_grad reads the
// gradient and, with skip_zeros, marks the blocks holding a nonzero gradient;
// load_rest reads the other inputs -- with skip_zeros only for those blocks (an
// all-zero block is neither read nor written).
template <int DT, int OPT, int BS, bool QUANT, bool SKIP>
__device__ __forceinline__ void load_grad(const StepArgs& a, int64_t base, int lane,
                                          TileRaw<DT, OPT, BS, QUANT>& r) {
    using L = Layout<BS>;
    using R = TileRaw<DT, OPT, BS, QUANT>;
    using Raw4 = typename Elem<DT>::Raw4;
    using T = typename Elem<DT>::T;
#pragma unroll
    for (int q = 0; q < R::NQ; ++q) {
        const Raw4 gv = ld_stream(reinterpret_cast<const Raw4*>(reinterpret_cast<const T*>(a.g) + L::elem(base, lane, q)));
#pragma unroll
        for (int i = 0; i < R::PW; ++i) r.g[q][i] = gv[i];
    }
    r.live = (1u << R::BPT) - 1u;
    if constexpr (SKIP) {
        r.live = 0;
#pragma unroll
        for (int b = 0; b < R::BPT; ++b) {
            bool nz = false;
#pragma unroll
            for (int qq = 0; qq < L::QPB; ++qq)
#pragma unroll
                for (int i = 0; i < R::PW; ++i) nz = nz || word_nonzero<DT>(r.g[b * L::QPB + qq][i]);
            if (wave_any(nz)) r.live |= 1u << b;
        }
    }
}

// Loads complete in issue order, so the inputs a tile consumes first go out first:
// the states (codes and absmax, or fp32 states), then p -- unless the state update
// itself reads p (decay folded into the gradient), when p goes first.
template <int OPT> struct StateReadsP {
    static constexpr bool v = OPT == kMomentum || OPT == kRmsprop || OPT == kAdagrad;
};

template <int DT, int OPT, int BS, bool QUANT, bool SKIP>
__device__ __forceinline__ void load_params(const StepArgs& a, int64_t base, int lane,
                                            TileRaw<DT, OPT, BS, QUANT>& r) {
    using L = Layout<BS>;
    using R = TileRaw<DT, OPT, BS, QUANT>;
    using Raw4 = typename Elem<DT>::Raw4;
    using T = typename Elem<DT>::T;
#pragma unroll
    for (int q = 0; q < R::NQ; ++q) {
        if (SKIP && !((r.live >> (q / L::QPB)) & 1u)) continue;          // wave-uniform
        const Raw4 pv = ld_stream(reinterpret_cast<const Raw4*>(reinterpret_cast<const T*>(a.p) + L::elem(base, lane, q)));
#pragma unroll
        for (int i = 0; i < R::PW; ++i) r.p[q][i] = pv[i];
    }
}

// BSA: the size of the blocks the absmax arrays index -- BS itself, or 2048 when the
// tile is one wave's half of a 2048-element block (see step_pairs).
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool WITHP = true, int BSA = BS>
__device__ __forceinline__ void load_rest(const StepArgs& a, int64_t base, int lane,
                                          TileRaw<DT, OPT, BS, QUANT>& r) {
    using L = Layout<BS>;
    using R = TileRaw<DT, OPT, BS, QUANT>;
    const int64_t blk0 = base / BSA;
    if constexpr (StateReadsP<OPT>::v) load_params<DT, OPT, BS, QUANT, SKIP>(a, base, lane, r);
#pragma unroll
    for (int k = 0; k < R::NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const int64_t eo = Slot<OPT>::elem_off(k, a.n);
        if constexpr (QUANT) {
            const uint8_t* cp = reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int q = 0; q < R::NQ; ++q) {
                if (SKIP && !((r.live >> (q / L::QPB)) & 1u)) continue;
                r.code[k][q] = ld_stream(reinterpret_cast<const uint32_t*>(cp + L::elem(base, lane, q)));
            }
            const float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
#pragma unroll
            for (int b = 0; b < R::BPT; ++b)
                r.A[k][b] = (!SKIP || ((r.live >> b) & 1u)) ? gbl(am)[blk0 + b] : 0.0f;
        } else {
            const float* fp = reinterpret_cast<const float*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int q = 0; q < R::NQ; ++q) {
                if (SKIP && !((r.live >> (q / L::QPB)) & 1u)) continue;
                r.fst[k][q] = ld_stream(reinterpret_cast<const f32x4*>(fp + L::elem(base, lane, q)));
            }
#pragma unroll
            for (int b = 0; b < R::BPT; ++b) r.A[k][b] = 0.0f;
        }
    }
    if constexpr (!StateReadsP<OPT>::v && WITHP) load_params<DT, OPT, BS, QUANT, SKIP>(a, base, lane, r);
}

template <int DT, int OPT, int BS, bool QUANT, bool SKIP, int BSA = BS>
__device__ __forceinline__ void load_tile(const StepArgs& a, int64_t base, int lane,
                                          TileRaw<DT, OPT, BS, QUANT>& r) {
    load_grad<DT, OPT, BS, QUANT, SKIP>(a, base, lane, r);
    load_rest<DT, OPT, BS, QUANT, SKIP, true, BSA>(a, base, lane, r);
}

// A wave pair's exchange of its halves' partial block maxima (see step_pairs): slot
// [iteration parity][wave][state].
typedef float PairExchange[2][kWavesPerGroup][4];

// Compute and store one full tile from its raw inputs.  PAIRX: the tile is one wave's
// half of a 2048-element block (BS = 1024, one block per tile); the block's absmax is
// formed with the partner wave's half through xch (one workgroup barrier) before the
// states are encoded, and only the first half stores it.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool FAST, bool PAIRX = false>
__device__ __forceinline__ void process_tile(const StepArgs& a, const MapLDS& M1, const MapLDS& M2,
                                             int64_t base, int lane, const TileRaw<DT, OPT, BS, QUANT>& r,
                                             PairExchange* xch = nullptr, int parity = 0) {
    using L = Layout<BS>;
    constexpr int NQ = L::NQ, BPT = L::BPT, QPB = L::QPB;
    constexpr int NS = NumStates<OPT>::v;
    static_assert(!PAIRX || (BS == 1024 && QUANT && !SKIP && !UNORM), "pair tiles: half of a 2048 block");
    const int64_t n = a.n;
    const int64_t blk0 = base / (PAIRX ? 2048 : BS);

    float pf[NQ][4], st[NS][NQ][4], dl[NQ][4];
    bool live[NQ][4];
    bool any_live[BPT];
#pragma unroll
    for (int b = 0; b < BPT; ++b) any_live[b] = false;
    constexpr bool ROOT = HasRoot<OPT>::v;
    constexpr bool EARLY = !SKIP && !UNORM;     // nothing waits on the block: store p per quad

#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (SKIP && !((r.live >> (q / QPB)) & 1u)) {
            // a block without a nonzero gradient: nothing was read, nothing is written
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pf[q][i] = 0.0f;
                dl[q][i] = 0.0f;
                live[q][i] = false;
#pragma unroll
                for (int k = 0; k < NS; ++k) st[k][q][i] = 0.0f;
            }
            continue;
        }
        float gq[4];
        widen_words<DT>(r.p[q], pf[q]);
        widen_words<DT>(r.g[q], gq);
        // decode this quad's states
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int slot = Slot<OPT>::which(k);
            const float* Q = slot ? M2.Q : M1.Q;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (QUANT) st[k][q][i] = Q[(r.code[k][q] >> (8 * i)) & 0xffu] * r.A[k][q / QPB];
                else st[k][q][i] = r.fst[k][q][i];
            }
        }
        // element updates (root optimizers: the new states first, then the step)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool skip = SKIP && (gq[i] == 0.0f);   // raw gradient; -0 counts as zero
            live[q][i] = !skip;
            any_live[q / QPB] = any_live[q / QPB] || live[q][i];
            float s3[3] = {st[0][q][i], NS > 1 ? st[NS > 1 ? 1 : 0][q][i] : 0.0f,
                           NS > 2 ? st[NS > 2 ? 2 : 0][q][i] : 0.0f};
            if constexpr (ROOT) {
                moments<OPT>(a.s, pf[q][i], gq[i], s3);
            } else {
                float d;
                update_elem<OPT>(a.s, pf[q][i], gq[i], s3, d);
                dl[q][i] = live[q][i] ? d : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < NS; ++k) st[k][q][i] = live[q][i] ? s3[k] : st[k][q][i];
        }
        bool applied = false;      // uniform: the new parameters are formed (in pf[q] or pw)
        bool packed = false;       // uniform: they are in pw, already rounded and packed
        uint32_t pw[2] = {0u, 0u};
        if constexpr (ROOT) {
            // The unscaled square root is exact unless a second moment of the quad lies
            // in (0, 2^-96); then the quad takes the general one (same bits either way).
            const bool any_tiny = wave_any(quad_needs_scaling(st[RootState<OPT>::v][q]));
            if constexpr (EARLY && DT != kF32) {
                // 16-bit parameters: the step from the hardware estimates gives the
                // stored parameter whenever the rounding test shows that no error
                // within the estimate's bound changes its 16-bit rounding; the quad
                // otherwise recomputes the step exactly (the same bits either way).
                if (OPT == kAdemamix && a.s.fast_root && !any_tiny) {
                    // three states: per element, the form with the fewest live values
                    float z[4];
                    bool unsure = false;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float s3[3] = {st[0][q][i], NS > 1 ? st[NS > 1 ? 1 : 0][q][i] : 0.0f,
                                             NS > 2 ? st[NS > 2 ? 2 : 0][q][i] : 0.0f};
                        const float d = root_delta_estimate<OPT>(a.s, pf[q][i], gq[i], s3);
                        const float pd = decayed<OPT>(a.s, pf[q][i]);
                        z[i] = pd - d;
                        unsure |= !rounds_alike<DT>(pd, d);
                    }
                    if (!wave_any(unsure)) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) pf[q][i] = z[i];
                        applied = true;
                    }
                } else if (a.s.fast_root && !any_tiny) {
                    bool sure = true;
                    uint32_t emax = 0;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float d[2], pd[2];
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const int i = 2 * h + j;
                            const float s3[3] = {st[0][q][i], NS > 1 ? st[NS > 1 ? 1 : 0][q][i] : 0.0f,
                                                 NS > 2 ? st[NS > 2 ? 2 : 0][q][i] : 0.0f};
                            d[j] = root_delta_estimate<OPT>(a.s, pf[q][i], gq[i], s3);
                            pd[j] = decayed<OPT>(a.s, pf[q][i]);
                        }
                        sure = pair_rounds_alike<DT>(pd[0], d[0], pd[1], d[1], pw[h], emax) && sure;
                    }
                    sure = sure && emax < 0x7F800000u;
                    if (!wave_any(!sure)) {
                        applied = true;
                        packed = true;
                    }
                }
            }
            auto deltas = [&](auto unscaled) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s3[3] = {st[0][q][i], NS > 1 ? st[NS > 1 ? 1 : 0][q][i] : 0.0f,
                                         NS > 2 ? st[NS > 2 ? 2 : 0][q][i] : 0.0f};
                    const float d = root_delta<OPT, decltype(unscaled)::value>(a.s, pf[q][i], gq[i], s3);
                    dl[q][i] = live[q][i] ? d : 0.0f;
                }
            };
            if (!applied) {
                if (any_tiny) deltas(std::false_type{});
                else deltas(std::true_type{});
            }
        }
        if constexpr (EARLY) {
            if (packed) {
                if constexpr (DT != kF32) {
                    using Raw4 = typename Elem<DT>::Raw4;
                    Raw4 r;
                    r.x = pw[0];
                    r.y = pw[1];
                    st_stream(r, reinterpret_cast<Raw4*>(reinterpret_cast<typename Elem<DT>::T*>(a.p) +
                                                         L::elem(base, lane, q)));
                }
            } else {
                if (!applied) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) pf[q][i] = apply_step<OPT>(a.s, pf[q][i], dl[q][i]);
                }
                store4<DT>(a.p, L::elem(base, lane, q), pf[q]);
            }
        }
    }

    // ---- per block: is anything written, and the cap of the update norm
    bool write[BPT];
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        write[b] = !SKIP || wave_any(any_live[b]);
        if constexpr (UNORM) {
            double su = 0.0, sp = 0.0;
#pragma unroll
            for (int qq = 0; qq < QPB; ++qq)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = b * QPB + qq;
                    const float d2 = dl[q][i] * dl[q][i];
                    const float p2 = pf[q][i] * pf[q][i];
                    su += (double)d2;
                    sp += (double)p2;
                }
            su = wave_sum_f64(su);
            sp = wave_sum_f64(sp);
            const double U = sqrt(su), P = sqrt(sp);
            const double lim = (double)a.s.max_unorm * P;
            if (U > lim) {
                const float clip = (float)(lim / U);
#pragma unroll
                for (int qq = 0; qq < QPB; ++qq)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dl[b * QPB + qq][i] = dl[b * QPB + qq][i] * clip;
            }
        }
    }

    if constexpr (SKIP || UNORM) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (!write[q / QPB]) continue;                 // wave-uniform
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[q][i] = live[q][i] ? apply_step<OPT>(a.s, pf[q][i], dl[q][i]) : pf[q][i];
            store4<DT>(a.p, L::elem(base, lane, q), pf[q]);
        }
    }

    // ---- pair tiles: the block absmax over both halves
    float Apair[NS];
    if constexpr (PAIRX) {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            float x = 0.0f;
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) x = fmaxf(x, fabsf(st[k][q][i]));
            Apair[k] = wave_max_nonneg(x);
            if (lane == 0) (*xch)[parity][wave][k] = Apair[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const float other = __int_as_float(__builtin_amdgcn_readfirstlane(
                __float_as_int((*xch)[parity][wave ^ 1][k])));
            Apair[k] = __int_as_float(max(__float_as_int(Apair[k]), __float_as_int(other)));
        }
    }

    // ---- states: new absmax and codes (8-bit) or fp32 values
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const int64_t eo = Slot<OPT>::elem_off(k, n);
        if constexpr (QUANT) {
            uint32_t w[NQ];
            float Al;
            if constexpr (PAIRX) {
                Al = Apair[k];
                if (k == RootState<OPT>::v && HasRoot<OPT>::v)
                    encode_tile_given<BS, FAST, true>(slot ? M2 : M1, st[k], w, Al);
                else
                    encode_tile_given<BS, FAST, false>(slot ? M2 : M1, st[k], w, Al);
            } else if (k == RootState<OPT>::v && HasRoot<OPT>::v) {      // a second moment: never negative
                encode_tile<BS, FAST, true>(slot ? M2 : M1, st[k], w, Al);
            } else {
                encode_tile<BS, FAST, false>(slot ? M2 : M1, st[k], w, Al);
            }
            float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
            uint8_t* cp = reinterpret_cast<uint8_t*>(slot ? a.s2 : a.s1) + eo;
            uint32_t wmask = 0;
#pragma unroll
            for (int b = 0; b < BPT; ++b) wmask |= write[b] ? 1u << b : 0u;
            if constexpr (PAIRX) {
                if ((threadIdx.x & 64) == 0 && lane == 0) gbl(am)[blk0] = Al;     // the pair's first half
            } else {
                store_absmax<BPT>(am, blk0, lane, Al, wmask);
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (write[q / QPB]) store_code_word<true>(cp, L::elem(base, lane, q), n, w[q]);
        } else {
            float* fp = reinterpret_cast<float*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (!write[q / QPB]) continue;
                const f32x4 v = {st[k][q][0], st[k][q][1], st[k][q][2], st[k][q][3]};
                st_stream(v, reinterpret_cast<f32x4*>(fp + L::elem(base, lane, q)));
            }
        }
    }
}

// ---------------------------------------------------------------- guarded tiles

// Lane j's value of v (wave-uniform).
__device__ __forceinline__ float lane_value(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// One quad of a quad-at-a-time tile: the loads (VEC: one vector access per array;
// otherwise element-wise, values past n read as zero), the decoded states and the
// element updates, exactly as a full tile computes them.  Returns the live
// elements as bits 0-3.  Both passes of guarded_tile call it, so the second pass
// recomputes what the first one saw.
template <int DT, int OPT, bool QUANT, bool SKIP, bool VEC>
__device__ __forceinline__ uint32_t guarded_quad(const StepArgs& a, const MapLDS& M1, const MapLDS& M2, int64_t e,
                                                 const float (&A)[NumStates<OPT>::v], float (&pv)[4],
                                                 float (&st)[NumStates<OPT>::v][4], float (&dl)[4]) {
    constexpr int NS = NumStates<OPT>::v;
    const int64_t n = a.n;
    float gv[4];
    if constexpr (VEC) {
        load4<DT>(a.p, e, pv);
        load4<DT>(a.g, e, gv);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = e + i < n;
            pv[i] = valid ? load1<DT>(a.p, e + i) : 0.0f;
            gv[i] = valid ? load1<DT>(a.g, e + i) : 0.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const int64_t eo = Slot<OPT>::elem_off(k, n);
        if constexpr (QUANT) {
            const uint8_t* cp = reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + eo;
            const float* Q = slot ? M2.Q : M1.Q;
            if constexpr (VEC) {
                const uint32_t w = ld_stream(reinterpret_cast<const uint32_t*>(cp + e));
#pragma unroll
                for (int i = 0; i < 4; ++i) st[k][i] = Q[(w >> (8 * i)) & 0xffu] * A[k];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) st[k][i] = e + i < n ? Q[gbl(cp)[e + i]] * A[k] : 0.0f;
            }
        } else {
            const float* fp = reinterpret_cast<const float*>(slot ? a.s2 : a.s1) + eo;
            if constexpr (VEC) {
                const f32x4 v = ld_stream(reinterpret_cast<const f32x4*>(fp + e));
#pragma unroll
                for (int i = 0; i < 4; ++i) st[k][i] = v[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) st[k][i] = e + i < n ? gbl(fp)[e + i] : 0.0f;
            }
        }
    }
    uint32_t livem = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool valid = VEC || e + i < n;
        const bool skip = SKIP && (gv[i] == 0.0f);
        const bool live = valid && !skip;
        livem |= live ? 1u << i : 0u;
        float s3[3] = {st[0][i], NS > 1 ? st[NS > 1 ? 1 : 0][i] : 0.0f, NS > 2 ? st[NS > 2 ? 2 : 0][i] : 0.0f};
        float d;
        update_elem<OPT>(a.s, pv[i], gv[i], s3, d);
        dl[i] = live ? d : 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) st[k][i] = live ? s3[k] : st[k][i];
    }
    return livem;
}

// A tile one quad at a time: ragged or misaligned tiles (VEC false: element-wise
// accesses), and every full tile when the maps need the binary-search encoder (VEC
// true), whose register footprint would otherwise set the whole kernel's.  Pass 1
// reads the inputs and forms what each block needs (new absmax, whether anything
// is written, update norms) as its last quad goes by; pass 2 reads them again,
// recomputes, encodes and stores.  The results are those of a full tile holding
// the same values (elements past n count as zeros and are never written).  The
// loops stay rolled and per-block values live in lane b of a register, so the
// path adds little to the kernel's register footprint.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool FAST, bool VEC>
__device__ __forceinline__ void guarded_tile(const StepArgs& a, const MapLDS& M1, const MapLDS& M2,
                                             int64_t base, int lane) {
    using L = Layout<BS>;
    constexpr int NQ = L::NQ, BPT = L::BPT, QPB = L::QPB;
    constexpr int NS = NumStates<OPT>::v;
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;
    // An opaque copy of the lane index: without it the compiler hoists this path's
    // lane-derived addresses out of the tile loop, and they then occupy registers
    // through the full-tile path as well.
    asm volatile("" : "+v"(lane));

    // lane b: block b's old absmax, new absmax with its reciprocal and prescale, clip factor
    float A0v[NS], Av[NS], rv[NS], cv[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const float* am = (Slot<OPT>::which(k) ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
        A0v[k] = (QUANT && lane < BPT && blk0 + lane < a.nb) ? gbl(am)[blk0 + lane] : 0.0f;
        Av[k] = 0.0f;
        rv[k] = 0.0f;
        cv[k] = 1.0f;
    }
    float clipv = 1.0f;
    uint32_t wmask = 0, cmask = 0;     // blocks written / clipped (uniform)

    if constexpr (QUANT || SKIP || UNORM) {
        float mcur[NS];
        uint32_t anycur = 0;
        double su = 0.0, sp = 0.0;
#pragma unroll
        for (int k = 0; k < NS; ++k) mcur[k] = 0.0f;
#pragma unroll 1
        for (int q = 0; q < NQ; ++q) {
            const int qb = q / QPB;
            float Ab[NS], pv[4], st[NS][4], dl[4];
#pragma unroll
            for (int k = 0; k < NS; ++k) Ab[k] = lane_value(A0v[k], qb);
            anycur |= guarded_quad<DT, OPT, QUANT, SKIP, VEC>(a, M1, M2, L::elem(base, lane, q), Ab, pv, st, dl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int k = 0; k < NS; ++k) mcur[k] = fmaxf(mcur[k], fabsf(st[k][i]));
                if constexpr (UNORM) {
                    const float d2 = dl[i] * dl[i];
                    const float p2 = pv[i] * pv[i];
                    su += (double)d2;
                    sp += (double)p2;
                }
            }
            if (q % QPB != QPB - 1) continue;               // block qb not complete yet
            if (blk0 + qb < a.nb && (!SKIP || wave_any(anycur != 0u))) wmask |= 1u << qb;
            if constexpr (UNORM) {
                const double U = sqrt(wave_sum_f64(su)), P = sqrt(wave_sum_f64(sp));
                const double lim = (double)a.s.max_unorm * P;
                if (U > lim) {
                    cmask |= 1u << qb;
                    clipv = lane == qb ? (float)(lim / U) : clipv;
                }
            }
            if constexpr (QUANT) {
#pragma unroll
                for (int k = 0; k < NS; ++k) {
                    const float u = wave_max_nonneg(mcur[k]);
                    float ru, cu;
                    block_recip(u, ru, cu);
                    Av[k] = lane == qb ? u : Av[k];
                    rv[k] = lane == qb ? ru : rv[k];
                    cv[k] = lane == qb ? cu : cv[k];
                    mcur[k] = 0.0f;
                }
            }
            anycur = 0;
            su = 0.0;
            sp = 0.0;
        }
    } else {
#pragma unroll
        for (int b = 0; b < BPT; ++b)
            if (blk0 + b < a.nb) wmask |= 1u << b;
    }

#pragma unroll 1
    for (int q = 0; q < NQ; ++q) {
        const int qb = q / QPB;
        if (!((wmask >> qb) & 1u)) continue;                 // wave-uniform
        const int64_t e = L::elem(base, lane, q);
        float Ab[NS], pv[4], st[NS][4], dl[4];
#pragma unroll
        for (int k = 0; k < NS; ++k) Ab[k] = lane_value(A0v[k], qb);
        const uint32_t livem = guarded_quad<DT, OPT, QUANT, SKIP, VEC>(a, M1, M2, e, Ab, pv, st, dl);
        if constexpr (UNORM) {
            if ((cmask >> qb) & 1u) {
                const float c = lane_value(clipv, qb);
#pragma unroll
                for (int i = 0; i < 4; ++i) dl[i] = dl[i] * c;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = ((livem >> i) & 1u) ? apply_step<OPT>(a.s, pv[i], dl[i]) : pv[i];
        if constexpr (VEC) {
            store4<DT>(a.p, e, pv);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < n) store1<DT>(a.p, e + i, pv[i]);
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int slot = Slot<OPT>::which(k);
            const int64_t eo = Slot<OPT>::elem_off(k, n);
            if constexpr (QUANT) {
                const float rb = lane_value(rv[k], qb), cb = lane_value(cv[k], qb);
                uint32_t w = 0;
                if (FAST && table_recip_ok(rb)) {                      // uniform
                    const float rs = rb * kEncScale;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w |= encode<true>(slot ? M2 : M1, (st[k][i] * cb) * rs) << (8 * i);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) w |= encode<false>(slot ? M2 : M1, (st[k][i] * cb) * rb) << (8 * i);
                }
                store_code_word<VEC>(reinterpret_cast<uint8_t*>(slot ? a.s2 : a.s1) + eo, e, n, w);
            } else {
                float* fp = reinterpret_cast<float*>(slot ? a.s2 : a.s1) + eo;
                if constexpr (VEC) {
                    const f32x4 v = {st[k][0], st[k][1], st[k][2], st[k][3]};
                    st_stream(v, reinterpret_cast<f32x4*>(fp + e));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (e + i < n) gbl(fp)[e + i] = st[k][i];
                }
            }
        }
    }
    if constexpr (QUANT) {
        if (lane < BPT && ((wmask >> lane) & 1u)) {
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                float* am = (Slot<OPT>::which(k) ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
                gbl(am)[blk0 + lane] = Av[k];
            }
        }
    }
}

// ---------------------------------------------------------------- tile loop and kernel

// Index of this wave in the grid, as a scalar (wave-uniform) value.
__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Multi-tensor launches: the tensor holding global tile gt and the tile's index in
// it -- the last table entry whose first tile is <= gt, by binary search over the
// first-tile indices staged in LDS.  The table is constant while the kernel runs,
// so its entries are read through the constant address space (scalar loads).
#define BITOPT_CONSTANT __attribute__((address_space(4)))
__device__ __forceinline__ int64_t resolve_tile(const StepArgs& a0, const uint32_t* T0, int64_t gt, StepArgs& a) {
    int lo = 0, hi = a0.ntab - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)T0[mid] <= gt) lo = mid; else hi = mid - 1;
    }
    const BITOPT_CONSTANT TensorDesc* tab = (const BITOPT_CONSTANT TensorDesc*)a0.table;
    const BITOPT_CONSTANT TensorDesc& d = tab[__builtin_amdgcn_readfirstlane(lo)];
    a = a0;
    a.p = d.p; a.g = d.g; a.s1 = d.s1; a.s2 = d.s2; a.a1 = d.a1; a.a2 = d.a2;
    a.n = d.n; a.nb = d.nb; a.vec = d.vec;
    return gt - d.tile0;
}

template <int BS, bool MULTI>
__device__ __forceinline__ int64_t total_tiles(const StepArgs& a) {
    if constexpr (MULTI) return a.total_tiles;
    else return (a.n + Layout<BS>::TE - 1) / Layout<BS>::TE;
}

// The tiles of one wave: gt = first, first + stride, ...  A full tile issues all of
// its loads before any use; latency is hidden by the other waves of the CU.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool MULTI, bool FAST>
__device__ __forceinline__ void step_tiles(const StepArgs& a0, const MapLDS& M1, const MapLDS& M2,
                                           const uint32_t* T0) {
    constexpr int64_t TE = Layout<BS>::TE;
    // the binary-search encoder runs on the quad-at-a-time path (see guarded_tile)
    constexpr bool WHOLE = !QUANT || FAST;
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = total_tiles<BS, MULTI>(a0);
    for (int64_t gt = wave_id(); gt < ntiles; gt += stride) {
        StepArgs am;
        int64_t t = gt;
        if constexpr (MULTI) t = resolve_tile(a0, T0, gt, am);
        const StepArgs& a = MULTI ? am : a0;
        if (tile_full<BS>(a, t)) {
            if constexpr (WHOLE) {
                TileRaw<DT, OPT, BS, QUANT> x;
                load_tile<DT, OPT, BS, QUANT, SKIP>(a, t * TE, lane, x);
                process_tile<DT, OPT, BS, QUANT, SKIP, UNORM, FAST>(a, M1, M2, t * TE, lane, x);
            } else {
                guarded_tile<DT, OPT, BS, QUANT, SKIP, UNORM, FAST, true>(a, M1, M2, t * TE, lane);
            }
        } else {
            guarded_tile<DT, OPT, BS, QUANT, SKIP, UNORM, FAST, false>(a, M1, M2, t * TE, lane);
        }
    }
}

// B = 2048 by wave pairs (single tensor, no skip_zeros or max_unorm): waves 2j and
// 2j+1 of a group share block b0 + j, each holding four quads of it (the register
// footprint of a 1024-element tile rather than a 2048-element one, so more waves fit
// per SIMD).  Each wave computes its half; the halves' maxima meet in LDS across one
// workgroup barrier per iteration; each wave encodes and stores its own half.  A
// block that is ragged, or a tensor that is not aligned for the vector path, is
// taken whole by the pair's first wave on the quad-at-a-time path.  The loop bounds
// are uniform over the group, so every wave passes the same number of barriers.
template <int DT, int OPT, bool FAST>
__device__ __forceinline__ void step_pairs(const StepArgs& a, const MapLDS& M1, const MapLDS& M2,
                                           PairExchange* xch) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = wave & 1;
    int parity = 0;
    for (int64_t b0 = (int64_t)blockIdx.x * 2; b0 < a.nb; b0 += (int64_t)gridDim.x * 2) {
        const int64_t blk = b0 + (wave >> 1);
        const bool inb = blk < a.nb;
        // the same for both waves of the pair; the binary-search encoder (maps other than
        // the standard ones) always takes the quad-at-a-time path
        const bool full = FAST && inb && a.vec && (blk + 1) * 2048 <= a.n;
        if constexpr (FAST) {
            if (full) {
                const int64_t base = blk * 2048 + (int64_t)half * 1024;
                TileRaw<DT, OPT, 1024, true> x;
                load_tile<DT, OPT, 1024, true, false, 2048>(a, base, lane, x);
                process_tile<DT, OPT, 1024, true, false, false, true, true>(a, M1, M2, base, lane, x, xch, parity);
            }
        }
        if (!full) {
            __syncthreads();                      // the barrier of process_tile's exchange
            if (inb && half == 0) guarded_tile<DT, OPT, 2048, true, false, false, FAST, false>(a, M1, M2, blk * 2048, lane);
        }
        parity ^= 1;
    }
}

// skip_zeros, one tile per wave (single tensor, grid covering every tile): the
// gradient is read before the maps are staged, and a group none of whose tiles has
// a nonzero gradient ends there -- most groups of a sparse update do no more than
// read their gradients.
template <int DT, int OPT, int BS, bool QUANT, bool UNORM, int NMAPS>
__device__ __forceinline__ void step_one_tile_skip(const StepArgs& a, float* Q1, float* Q2, float* T1, float* T2,
                                                   uint8_t* B1, uint8_t* B2, uint32_t* vote) {
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_id();
    const int64_t ntiles = total_tiles<BS, false>(a);
    const bool full = t < ntiles && tile_full<BS>(a, t);
    TileRaw<DT, OPT, BS, QUANT> x;
    x.live = 0;
    if (full) load_grad<DT, OPT, BS, QUANT, true>(a, t * TE, lane, x);
    // ragged or misaligned tiles are taken as having work
    const bool work = full ? x.live != 0u : t < ntiles;
    if (!__syncthreads_or(work)) return;
    const MapLDS M1{Q1, T1, B1}, M2{Q2, T2, B2};
    bool fast = true;
    if constexpr (QUANT) fast = stage_maps<NMAPS, UnsignedState1<OPT>::v>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2, vote);
    if (!work) return;
    if (full) {
        if (!QUANT || fast) {
            load_rest<DT, OPT, BS, QUANT, true>(a, t * TE, lane, x);
            process_tile<DT, OPT, BS, QUANT, true, UNORM, true>(a, M1, M2, t * TE, lane, x);
        } else {
            guarded_tile<DT, OPT, BS, QUANT, true, UNORM, false, true>(a, M1, M2, t * TE, lane);
        }
    } else if (fast) {
        guarded_tile<DT, OPT, BS, QUANT, true, UNORM, true, false>(a, M1, M2, t * TE, lane);
    } else {
        guarded_tile<DT, OPT, BS, QUANT, true, UNORM, false, false>(a, M1, M2, t * TE, lane);
    }
}

// One tile per wave (single tensor, grid covering every tile), no skip_zeros: the
// gradient and the states of the tile are requested before the maps are staged (p
// after), so their HBM latency overlaps the staging loads and the barrier.  Used
// for fp32 parameters at B = 2048 (the largest tile, at four waves per SIMD), where
// it shortens the step by 4%; at B = 256 and for 16-bit parameters the extra
// registers held across the staging cost as much as the overlap gains.
template <int DT, int OPT, int BS, bool QUANT, bool UNORM, int NMAPS>
__device__ __forceinline__ void step_one_tile(const StepArgs& a, float* Q1, float* Q2, float* T1, float* T2,
                                              uint8_t* B1, uint8_t* B2, uint32_t* vote) {
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t t = wave_id();
    const int64_t ntiles = total_tiles<BS, false>(a);
    const bool full = t < ntiles && tile_full<BS>(a, t);
    TileRaw<DT, OPT, BS, QUANT> x;
    if (full) {
        load_grad<DT, OPT, BS, QUANT, false>(a, t * TE, lane, x);
        load_rest<DT, OPT, BS, QUANT, false, false>(a, t * TE, lane, x);
    }
    const MapLDS M1{Q1, T1, B1}, M2{Q2, T2, B2};
    bool fast = true;
    if constexpr (QUANT) fast = stage_maps<NMAPS, UnsignedState1<OPT>::v>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2, vote);
    if (t >= ntiles) return;
    if (full) {
        if (!QUANT || fast) {
            if constexpr (!StateReadsP<OPT>::v) load_params<DT, OPT, BS, QUANT, false>(a, t * TE, lane, x);
            process_tile<DT, OPT, BS, QUANT, false, UNORM, true>(a, M1, M2, t * TE, lane, x);
        } else {
            guarded_tile<DT, OPT, BS, QUANT, false, UNORM, false, true>(a, M1, M2, t * TE, lane);
        }
    } else if (fast) {
        guarded_tile<DT, OPT, BS, QUANT, false, UNORM, true, false>(a, M1, M2, t * TE, lane);
    } else {
        guarded_tile<DT, OPT, BS, QUANT, false, UNORM, false, false>(a, M1, M2, t * TE, lane);
    }
}

// Minimum resident waves per SIMD asked of the register allocator, for the 8-bit
// steps on 16-bit parameters at B = 256 without skip_zeros or max_unorm: AdEMAMix
// (three states) five, Adam six, Momentum and Lion eight -- each the most that fits
// without spilling, and measured faster than the allocator's own choice (AdEMAMix
// at six spills and runs 15% slower).  Every other instantiation keeps the
// allocator's choice.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM> struct MinWaves {
    static constexpr bool hot16 = DT != kF32 && BS == 256 && QUANT && !SKIP && !UNORM;
    static constexpr bool pair = BS == 2048 && QUANT && !SKIP && !UNORM && OPT == kAdam;
    static constexpr int v = pair ? 5 : !hot16 ? 1 : OPT == kAdemamix ? 5 : OPT == kAdam ? 6 : (OPT == kMomentum || OPT == kLion) ? 8 : 1;
};

// Steps whose 2048-element blocks are taken by wave pairs (step_pairs).
template <int BS, bool QUANT, bool SKIP, bool UNORM, bool MULTI> struct PairBlocks {
    static constexpr bool v = BS == 2048 && QUANT && !SKIP && !UNORM && !MULTI;
};

// One launch of the fused step: a single tensor (MULTI false: the launch arguments)
// or every tensor of a descriptor table (MULTI true).
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool MULTI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MinWaves<DT, OPT, BS, QUANT, SKIP, UNORM>::v)))
void k_step(StepArgs a) {
    constexpr int NMAPS = (OPT == kAdam || OPT == kAdemamix) ? 2 : 1;
    __shared__ float Q1[256], Q2[256], T1[256], T2[256];
    __shared__ __attribute__((aligned(16))) uint8_t B1[search::kNB];
    __shared__ __attribute__((aligned(16))) uint8_t B2[search::kNB];
    __shared__ uint32_t vote[kWavesPerGroup];
    __shared__ uint32_t T0[MULTI ? kMaxTableTensors : 1];   // first tiles (< 2^32 per launch)
    const MapLDS M1{Q1, T1, B1}, M2{Q2, T2, B2};
    if constexpr (PairBlocks<BS, QUANT, SKIP, UNORM, MULTI>::v) {
        __shared__ PairExchange xch[1];
        if (stage_maps<NMAPS, UnsignedState1<OPT>::v>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2, vote))
            step_pairs<DT, OPT, true>(a, M1, M2, xch);
        else
            step_pairs<DT, OPT, false>(a, M1, M2, xch);
        return;
    }
    if constexpr (MULTI) {
        // scalars the caller writes into device memory before each launch or graph replay
        if (a.sdev) a.s = *a.sdev;      // uniform
        const BITOPT_CONSTANT TensorDesc* tab = (const BITOPT_CONSTANT TensorDesc*)a.table;
        for (int i = threadIdx.x; i < a.ntab; i += kThreads) T0[i] = (uint32_t)tab[i].tile0;
        __syncthreads();
    }
    if constexpr (!MULTI && (SKIP || (BS == 2048 && DT == kF32))) {
        if ((int64_t)gridDim.x * kWavesPerGroup >= total_tiles<BS, false>(a)) {     // uniform
            if constexpr (SKIP) step_one_tile_skip<DT, OPT, BS, QUANT, UNORM, NMAPS>(a, Q1, Q2, T1, T2, B1, B2, vote);
            else step_one_tile<DT, OPT, BS, QUANT, UNORM, NMAPS>(a, Q1, Q2, T1, T2, B1, B2, vote);
            return;
        }
    }
    if constexpr (QUANT) {
        if (stage_maps<NMAPS, UnsignedState1<OPT>::v>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2, vote))
            step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, MULTI, true>(a, M1, M2, T0);
        else
            step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, MULTI, false>(a, M1, M2, T0);
    } else {
        step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, MULTI, false>(a, M1, M2, T0);
    }
}

// ---------------------------------------------------------------- codec kernels

struct CodecArgs {
    const void* x;       // quantize input
    void* out;           // dequantize output
    uint8_t* codes;
    float* absmax;
    const float* qmap;
    int64_t n;
    int64_t nb;
    int32_t vec;
};

template <int DT, int BS, bool FAST, bool FULL>
__device__ __forceinline__ void quant_tile(const CodecArgs& a, const MapLDS& M, int64_t base, int lane) {
    using L = Layout<BS>;
    constexpr int NQ = L::NQ;
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;
    float v[NQ][4];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t e = L::elem(base, lane, q);
        if constexpr (FULL) load4<DT>(a.x, e, v[q]);
        else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[q][i] = e + i < n ? load1<DT>(a.x, e + i) : 0.0f;
        }
    }
    uint32_t w[NQ];
    float Al;
    encode_tile<BS, FAST, false>(M, v, w, Al);
    uint32_t wmask = 0;
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) wmask |= (FULL || blk0 + b < a.nb) ? 1u << b : 0u;
    store_absmax<L::BPT>(a.absmax, blk0, lane, Al, wmask);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        if (FULL || blk0 + q / L::QPB < a.nb) store_code_word<FULL>(a.codes, L::elem(base, lane, q), n, w[q]);
}

// Quantize one tile with the binary-search encoder (maps without search tables): two
// passes holding one quad at a time -- the block maxima first, then each quad is read
// again and encoded -- so that this path, which only other maps take, does not raise
// the register count of the kernel's table path.  The same arithmetic as quant_tile.
template <int DT, int BS>
__device__ __forceinline__ void quant_tile_search(const CodecArgs& a, const MapLDS& M, int64_t base, int lane) {
    using L = Layout<BS>;
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;
    const bool full = a.vec && base + L::TE <= n;
    auto quad = [&](int q, float (&v)[4]) {
        const int64_t e = L::elem(base, lane, q);
        if (full) {
            load4<DT>(a.x, e, v);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = e + i < n ? load1<DT>(a.x, e + i) : 0.0f;
        }
    };
    float m[L::BPT];
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) {
        float x = 0.0f;
#pragma unroll 1
        for (int qq = 0; qq < L::QPB; ++qq) {
            float v[4];
            quad(b * L::QPB + qq, v);
#pragma unroll
            for (int i = 0; i < 4; ++i) x = fmaxf(x, fabsf(v[i]));
        }
        m[b] = x;
    }
    float u, ru, cu;
    block_absmax_lanes<L::BPT>(m, u, ru, cu);
    uint32_t wmask = 0;
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) wmask |= (blk0 + b < a.nb) ? 1u << b : 0u;
    store_absmax<L::BPT>(a.absmax, blk0, lane, u, wmask);
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) {
        if (!((wmask >> b) & 1u)) continue;                 // uniform
        const float rq = block_value<L::BPT>(ru, b), cq = block_value<L::BPT>(cu, b);
#pragma unroll 1
        for (int qq = 0; qq < L::QPB; ++qq) {
            const int q = b * L::QPB + qq;
            float v[4];
            quad(q, v);
            uint32_t x = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x |= encode<false>(M, (v[i] * cq) * rq) << (8 * i);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (full) store_code_word<true>(a.codes, L::elem(base, lane, q), n, x);
            else store_code_word<false>(a.codes, L::elem(base, lane, q), n, x);
        }
    }
}

template <int DT, int BS, bool FAST>
__device__ __forceinline__ void quant_tiles(const CodecArgs& a, const MapLDS& M) {
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + TE - 1) / TE;
    for (int64_t t = wave_id(); t < ntiles; t += nwaves) {
        const int64_t base = t * TE;
        if constexpr (!FAST) quant_tile_search<DT, BS>(a, M, base, lane);
        else if (a.vec && base + TE <= a.n) quant_tile<DT, BS, true, true>(a, M, base, lane);
        else quant_tile<DT, BS, true, false>(a, M, base, lane);
    }
}

template <int DT, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BS == 256 ? 8 : 1))) void k_quantize(CodecArgs a) {
    __shared__ float Q[256], T[256];
    __shared__ __attribute__((aligned(16))) uint8_t B[search::kNB];
    __shared__ uint32_t vote[kWavesPerGroup];
    const MapLDS M{Q, T, B};
    if (stage_maps<1>(a.qmap, nullptr, Q, nullptr, T, nullptr, B, nullptr, vote)) quant_tiles<DT, BS, true>(a, M);
    else quant_tiles<DT, BS, false>(a, M);
}

// out[i] = qmap[codes[i]] * absmax[i / BS], in the step kernels' tile layout: a wave
// owns 4 (B = 256) or 8 (B = 2048) quads, issues the code loads of all of them first,
// reads each quad's absmax once (uniform), then gathers, scales and stores.
template <int DT, int BS>
__device__ __forceinline__ void dequant_tile(const CodecArgs& a, const float* Q, int64_t base, int lane) {
    using L = Layout<BS>;
    constexpr int NQ = L::NQ;
    if (a.vec && base + L::TE <= a.n) {
        uint32_t w[NQ];
        float A[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) w[q] = ld_stream(reinterpret_cast<const uint32_t*>(a.codes + L::elem(base, lane, q)));
#pragma unroll
        for (int q = 0; q < NQ; ++q) A[q] = gbl(a.absmax)[(base + q * 256) / BS];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = Q[(w[q] >> (8 * i)) & 0xffu] * A[q];
            store4<DT>(a.out, L::elem(base, lane, q), v);
        }
    } else {
#pragma unroll 1
        for (int q = 0; q < NQ; ++q) {
            const int64_t e = L::elem(base, lane, q);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < a.n) store1<DT>(a.out, e + i, Q[gbl(a.codes)[e + i]] * gbl(a.absmax)[(e + i) / BS]);
        }
    }
}

template <int DT, int BS>
__global__ __launch_bounds__(kThreads) void k_dequantize(CodecArgs a) {
    __shared__ float Q[256];
    Q[threadIdx.x] = gbl(a.qmap)[threadIdx.x];
    __syncthreads();
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + TE - 1) / TE;
    for (int64_t t = wave_id(); t < ntiles; t += nwaves) dequant_tile<DT, BS>(a, Q, t * TE, lane);
}

}  // namespace bitopt
