// kernels.h -- gfx950 device code of libbitopt: the fused 8-bit block-wise
// optimizer step, its 32-bit (identity codec) twin and the block-wise codec.
//
// Work decomposition (CDNA4, wave64).  A wavefront owns a tile of NQ quads; quad q
// of lane l holds elements q*256 + 4l .. +3, so every load/store instruction of the
// wave covers one contiguous 256-element span (16 B/lane for fp32, 8 B/lane for
// 16-bit, 4 B/lane of codes) and carries the non-temporal hint.  Blocks of 256 are
// single quads (four per tile): their absmax comes from one reduce-scatter across
// the wave; a block of 2048 is a whole tile, reduced by DPP row shifts, row
// broadcasts and readlane.  Tiles are software-pipelined two deep.  The 256-entry
// codebooks sit in LDS; decoding is one LDS gather.  Encoding with a standard
// dynamic map is one bucket lookup (exponent and top mantissa bits of x) plus one
// comparison with an fp32 decision threshold, both in LDS; any other map falls
// back to a branch-free binary search plus one neighbour comparison.  Both give
// the nearest entry (fp32 distance, ties to the lower index).
//
// Arithmetic.  Each element operation is one IEEE fp32 operation in a fixed order
// (the build disables FMA contraction and keeps correctly rounded division and
// square root), so results do not depend on the tiling and are reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitopt_tables.h"   // generated: constant search tables of the standard maps
#include "search_layout.h"

namespace bitopt {

constexpr int kF32 = 0, kF16 = 1, kBF16 = 2;
constexpr int kAdam = 0, kAdemamix = 1, kMomentum = 2, kLion = 3;
constexpr int kThreads = 256;              // 4 waves per workgroup
constexpr int kWavesPerGroup = kThreads / 64;

// Per-step scalars, formed on the host in double and rounded once to fp32.
struct StepScalars {
    float lr, b1, b2, eps, wd;
    float omb1, omb2, ic1, rs2, decay;
    float b3t, omb3, alpha_t;
    float max_unorm;
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
};

template <int OPT> struct NumStates { static constexpr int v = OPT == kAdemamix ? 3 : (OPT == kAdam ? 2 : 1); };

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
template <class T> __device__ __forceinline__ T ld_stream(const T* p) {
    if constexpr (BITOPT_NONTEMPORAL) return __builtin_nontemporal_load(p);
    else return *p;
}
template <class T> __device__ __forceinline__ void st_stream(T v, T* p) {
    if constexpr (BITOPT_NONTEMPORAL) __builtin_nontemporal_store(v, p);
    else *p = v;
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
    const typename Elem<DT>::T x = reinterpret_cast<const typename Elem<DT>::T*>(base)[e];
    if constexpr (DT == kF32) return x;
    else return widen<DT>((uint32_t)x);
}
template <int DT> __device__ __forceinline__ void store1(void* base, int64_t e, float v) {
    if constexpr (DT == kF32) reinterpret_cast<float*>(base)[e] = v;
    else reinterpret_cast<uint16_t*>(base)[e] = (uint16_t)narrow<DT>(v);
}

// ---------------------------------------------------------------- wave reductions

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    // Lanes whose source lane is outside the pattern, or whose row is masked off,
    // read 0 (the identity of a max over non-negative values).
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Max over the 64 lanes of non-negative values; the result is wave-uniform.
// row_shr 1,2,4,8 leave each row's max in its lane 15; row_bcast15 and row_bcast31
// carry it across rows into lane 63, which is then read as a scalar.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, dpp_or_zero<0x111, 0xF>(v));
    v = fmaxf(v, dpp_or_zero<0x112, 0xF>(v));
    v = fmaxf(v, dpp_or_zero<0x114, 0xF>(v));
    v = fmaxf(v, dpp_or_zero<0x118, 0xF>(v));
    v = fmaxf(v, dpp_or_zero<0x142, 0xA>(v));
    v = fmaxf(v, dpp_or_zero<0x143, 0xC>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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
__device__ __forceinline__ float dpp_rot(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float row_max_nonneg(float v) {
    v = fmaxf(v, dpp_rot<0x128>(v));    // row_ror 8, 4, 2, 1
    v = fmaxf(v, dpp_rot<0x124>(v));
    v = fmaxf(v, dpp_rot<0x122>(v));
    v = fmaxf(v, dpp_rot<0x121>(v));
    return v;
}

// ---------------------------------------------------------------- codebook search

// Nearest entry of a sorted 256-entry map Q (in LDS) to x: the largest i in
// [0, 254] with Q[i] <= x (or 0), then i+1 if it is strictly closer in fp32.
__device__ __forceinline__ uint32_t nearest_code(const float* Q, float x) {
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

// Nearest code of x.  FAST (standard maps): one bucket lookup and one threshold
// comparison, code = bkt[idx(x)] + (x >= tau[bkt[idx(x)]]), which equals the
// nearest-entry rule for every finite x.  Otherwise the binary search above.
template <bool FAST>
__device__ __forceinline__ uint32_t encode(const MapLDS& m, float x) {
    if constexpr (FAST) {
        using namespace search;
        const uint32_t bits = __float_as_uint(x);
        const uint32_t key = (bits >> (23 - kM)) & ((1u << (8 + kM)) - 1u);
        const uint32_t b = min(max(key, (uint32_t)kKLO), (uint32_t)kKHI) - (uint32_t)kKLO;
        const uint32_t idx = (uint32_t)kNBH + (b ^ (uint32_t)((int32_t)bits >> 31));
        const uint32_t c = m.bkt[idx];
        return c + (x >= m.tau[c] ? 1u : 0u);
    } else {
        return nearest_code(m.Q, x);
    }
}

// Stage up to two codebooks into LDS.  Every thread of the (256-thread) group
// copies one entry and checks it against the two standard maps; the group takes
// the table path only when every staged map is a standard one.  Returns that
// choice (uniform over the group).
template <int NMAPS>
__device__ __forceinline__ bool stage_maps(const float* q1, const float* q2, float* Q1, float* Q2,
                                           float* T1, float* T2, uint8_t* B1, uint8_t* B2) {
    const int tid = threadIdx.x;
    const float* src[2] = {q1, q2};
    float* Q[2] = {Q1, Q2};
    float* T[2] = {T1, T2};
    uint8_t* Bk[2] = {B1, B2};
    int which[2] = {-1, -1};
#pragma unroll
    for (int k = 0; k < NMAPS; ++k) {
        const uint32_t v = __float_as_uint(src[k][tid]);
        Q[k][tid] = __uint_as_float(v);
        if (__syncthreads_and(v == kStdQ0[tid])) which[k] = 0;
        else if (__syncthreads_and(v == kStdQ1[tid])) which[k] = 1;
    }
    bool fast = true;
#pragma unroll
    for (int k = 0; k < NMAPS; ++k) fast = fast && which[k] >= 0;
    if (fast) {
#pragma unroll
        for (int k = 0; k < NMAPS; ++k) {
            const uint32_t* tsrc = which[k] ? kStdTau1 : kStdTau0;
            const uint32_t* bsrc = reinterpret_cast<const uint32_t*>(which[k] ? kStdBucket1 : kStdBucket0);
            T[k][tid] = __uint_as_float(tsrc[tid]);
            uint32_t* bdst = reinterpret_cast<uint32_t*>(Bk[k]);
            for (int i = tid; i < search::kNB / 4; i += kThreads) bdst[i] = bsrc[i];
        }
    }
    __syncthreads();
    return fast;
}

// ---------------------------------------------------------------- optimizer updates

// One element of one step.  st[] holds the decoded states on entry and the new
// states on exit; the parameter step delta is returned through d.
// Adam/AdamW: st = {m, v};  AdEMAMix: st = {m1, m2, nu};  Momentum: {buf};  Lion: {m}.
template <int OPT>
__device__ __forceinline__ void update_elem(const StepScalars& s, float p, float g, float st[3], float& d) {
    float t1, t2;
    if constexpr (OPT == kAdam) {
        float m = st[0], v = st[1];
        t1 = s.b1 * m; t2 = s.omb1 * g; m = t1 + t2;
        const float gg = g * g;
        t1 = s.b2 * v; t2 = s.omb2 * gg; v = t1 + t2;
        float den = sqrtf(v) * s.rs2;
        den = den + s.eps;
        const float mh = m * s.ic1;
        const float u = mh / den;
        d = s.lr * u;
        st[0] = m; st[1] = v;
    } else if constexpr (OPT == kAdemamix) {
        float m1 = st[0], m2 = st[1], nu = st[2];
        t1 = s.b1 * m1; t2 = s.omb1 * g; m1 = t1 + t2;
        t1 = s.b3t * m2; t2 = s.omb3 * g; m2 = t1 + t2;
        const float gg = g * g;
        t1 = s.b2 * nu; t2 = s.omb2 * gg; nu = t1 + t2;
        float den = sqrtf(nu) * s.rs2;
        den = den + s.eps;
        t1 = m1 * s.ic1; t2 = s.alpha_t * m2;
        const float num = t1 + t2;
        const float u = num / den;
        d = s.lr * u;
        st[0] = m1; st[1] = m2; st[2] = nu;
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

template <int OPT>
__device__ __forceinline__ float apply_step(const StepScalars& s, float p, float d) {
    if constexpr (OPT == kMomentum) return p - d;
    else { const float pd = p * s.decay; return pd - d; }
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
// partial maxima m[b] (non-negative).  Results are wave-uniform.
// One block per tile: a wave max.  Four blocks per tile: a reduce-scatter -- two
// exchanges between lane halves and row pairs leave row r with the partial max of
// block r, a row reduction completes it, one reciprocal serves all four blocks, and
// each block's pair is then read from its row's first lane.
template <int BPT>
__device__ __forceinline__ void block_absmax(const float (&m)[BPT], float (&A)[BPT], float (&r)[BPT]) {
    if constexpr (BPT == 1) {
        A[0] = wave_max_nonneg(m[0]);
        r[0] = (A[0] == 0.0f) ? 0.0f : 1.0f / A[0];
    } else {
        static_assert(BPT == 4, "tiles hold one or four blocks");
        const int lane = threadIdx.x & 63;
        const bool hi = lane >= 32;
        const bool odd = (lane >> 4) & 1;
        // lanes 0-31 keep blocks 0,1 and lanes 32-63 blocks 2,3
        const float s0 = hi ? m[0] : m[2], s1 = hi ? m[1] : m[3];
        const float k0 = hi ? m[2] : m[0], k1 = hi ? m[3] : m[1];
        const float w0 = fmaxf(k0, __shfl_xor(s0, 32, 64));
        const float w1 = fmaxf(k1, __shfl_xor(s1, 32, 64));
        // even rows keep the first of the pair, odd rows the second: row r -> block r
        const float s = odd ? w0 : w1, k = odd ? w1 : w0;
        const float u = row_max_nonneg(fmaxf(k, __shfl_xor(s, 16, 64)));
        const float ru = (u == 0.0f) ? 0.0f : 1.0f / u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            A[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), 16 * b));
            r[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ru), 16 * b));
        }
    }
}

// The NQ code words (4 codes each) of a lane from a code array.
template <int BS, bool FULL>
__device__ __forceinline__ void load_codes(const uint8_t* cp, int64_t base, int lane, int64_t n, uint32_t w[]) {
    using L = Layout<BS>;
#pragma unroll
    for (int q = 0; q < L::NQ; ++q) {
        const int64_t e = L::elem(base, lane, q);
        if constexpr (FULL) {
            w[q] = ld_stream(reinterpret_cast<const uint32_t*>(cp + e));
        } else {
            uint32_t x = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) x |= (e + i < n ? (uint32_t)cp[e + i] : 0u) << (8 * i);
            w[q] = x;
        }
    }
}

template <bool FULL>
__device__ __forceinline__ void store_code_word(uint8_t* cp, int64_t e, int64_t n, uint32_t w) {
    if constexpr (FULL) {
        st_stream(w, reinterpret_cast<uint32_t*>(cp + e));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e + i < n) cp[e + i] = (uint8_t)(w >> (8 * i));
    }
}

// Encode the lane's values of one tile: per-block absmax (A, uniform), nearest
// codes of value * (1/A).  Quads of blocks past the end hold zeros.
template <int BS, bool FAST, int NQ>
__device__ __forceinline__ void encode_tile(const MapLDS& M, const float (&v)[NQ][4], uint32_t w[NQ],
                                            float (&A)[Layout<BS>::BPT]) {
    using L = Layout<BS>;
    float m[L::BPT], r[L::BPT];
#pragma unroll
    for (int b = 0; b < L::BPT; ++b) {
        float x = 0.0f;
#pragma unroll
        for (int qq = 0; qq < L::QPB; ++qq)
#pragma unroll
            for (int i = 0; i < 4; ++i) x = fmaxf(x, fabsf(v[b * L::QPB + qq][i]));
        m[b] = x;
    }
    block_absmax<L::BPT>(m, A, r);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const float rq = r[q / L::QPB];
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y = v[q][i] * rq;
            x |= encode<FAST>(M, y) << (8 * i);
        }
        w[q] = x;
    }
}

// ---------------------------------------------------------------- fused step tile

// Raw inputs of one lane for one tile, as loaded: parameter and gradient words,
// code words (8-bit) or fp32 states, and the tile's block absmax per state.
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
};

template <int DT, int PW>
__device__ __forceinline__ void load_words(const void* base, int64_t e, int64_t n, uint32_t (&w)[PW]) {
    if constexpr (DT == kF32) {
        const float* f = reinterpret_cast<const float*>(base);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = e + i < n ? __float_as_uint(f[e + i]) : 0u;
    } else {
        const uint16_t* h = reinterpret_cast<const uint16_t*>(base);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t lo = e + 2 * i < n ? (uint32_t)h[e + 2 * i] : 0u;
            const uint32_t hi = e + 2 * i + 1 < n ? (uint32_t)h[e + 2 * i + 1] : 0u;
            w[i] = lo | (hi << 16);
        }
    }
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

// Issue every load of one tile.  FULL: vector accesses (tile in range, buffers
// aligned); otherwise element-wise guarded accesses, out-of-range values zero.
template <int DT, int OPT, int BS, bool QUANT, bool FULL>
__device__ __forceinline__ void load_tile(const StepArgs& a, int64_t base, int lane,
                                          TileRaw<DT, OPT, BS, QUANT>& r) {
    using L = Layout<BS>;
    using R = TileRaw<DT, OPT, BS, QUANT>;
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;
#pragma unroll
    for (int q = 0; q < R::NQ; ++q) {
        const int64_t e = L::elem(base, lane, q);
        if constexpr (FULL) {
            using Raw4 = typename Elem<DT>::Raw4;
            const Raw4 pv = ld_stream(reinterpret_cast<const Raw4*>(reinterpret_cast<const typename Elem<DT>::T*>(a.p) + e));
            const Raw4 gv = ld_stream(reinterpret_cast<const Raw4*>(reinterpret_cast<const typename Elem<DT>::T*>(a.g) + e));
#pragma unroll
            for (int i = 0; i < R::PW; ++i) { r.p[q][i] = pv[i]; r.g[q][i] = gv[i]; }
        } else {
            load_words<DT, R::PW>(a.p, e, n, r.p[q]);
            load_words<DT, R::PW>(a.g, e, n, r.g[q]);
        }
    }
#pragma unroll
    for (int k = 0; k < R::NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const int64_t eo = Slot<OPT>::elem_off(k, n);
        if constexpr (QUANT) {
            load_codes<BS, FULL>(reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + eo, base, lane, n, r.code[k]);
            const float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
#pragma unroll
            for (int b = 0; b < R::BPT; ++b) r.A[k][b] = (FULL || blk0 + b < a.nb) ? am[blk0 + b] : 0.0f;
        } else {
            const float* fp = reinterpret_cast<const float*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int q = 0; q < R::NQ; ++q) {
                const int64_t e = L::elem(base, lane, q);
                if constexpr (FULL) {
                    r.fst[k][q] = ld_stream(reinterpret_cast<const f32x4*>(fp + e));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) r.fst[k][q][i] = e + i < n ? fp[e + i] : 0.0f;
                }
            }
#pragma unroll
            for (int b = 0; b < R::BPT; ++b) r.A[k][b] = 0.0f;
        }
    }
}

// Compute and store one tile from its raw inputs.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool FAST, bool FULL>
__device__ __forceinline__ void process_tile(const StepArgs& a, const MapLDS& M1, const MapLDS& M2,
                                             int64_t base, int lane, const TileRaw<DT, OPT, BS, QUANT>& r) {
    using L = Layout<BS>;
    constexpr int NQ = L::NQ, BPT = L::BPT, QPB = L::QPB;
    constexpr int NS = NumStates<OPT>::v;
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;

    float pf[NQ][4], st[NS][NQ][4], dl[NQ][4];
    bool live[NQ][4];
    bool any_live[BPT];
#pragma unroll
    for (int b = 0; b < BPT; ++b) any_live[b] = false;

#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t e = L::elem(base, lane, q);
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
                float v;
                if constexpr (QUANT) v = Q[(r.code[k][q] >> (8 * i)) & 0xffu] * r.A[k][q / QPB];
                else v = r.fst[k][q][i];
                st[k][q][i] = (FULL || e + i < n) ? v : 0.0f;
            }
        }
        // element updates
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = FULL || (e + i < n);
            const bool skip = SKIP && (gq[i] == 0.0f);   // raw gradient; -0 counts as zero
            live[q][i] = valid && !skip;
            any_live[q / QPB] = any_live[q / QPB] || live[q][i];
            float s3[3] = {st[0][q][i], NS > 1 ? st[NS > 1 ? 1 : 0][q][i] : 0.0f,
                           NS > 2 ? st[NS > 2 ? 2 : 0][q][i] : 0.0f};
            float d;
            update_elem<OPT>(a.s, pf[q][i], gq[i], s3, d);
            dl[q][i] = live[q][i] ? d : 0.0f;
#pragma unroll
            for (int k = 0; k < NS; ++k) st[k][q][i] = live[q][i] ? s3[k] : st[k][q][i];
        }
        if constexpr (!SKIP && !UNORM) {
            // nothing waits on the block: write this quad's parameters now
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[q][i] = live[q][i] ? apply_step<OPT>(a.s, pf[q][i], dl[q][i]) : pf[q][i];
            if constexpr (FULL) {
                store4<DT>(a.p, e, pf[q]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < n) store1<DT>(a.p, e + i, pf[q][i]);
            }
        }
    }

    // ---- per block: is anything written, and the cap of the update norm
    bool write[BPT];
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        write[b] = (FULL || blk0 + b < a.nb) && (!SKIP || wave_any(any_live[b]));
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
            const int64_t e = L::elem(base, lane, q);
#pragma unroll
            for (int i = 0; i < 4; ++i) pf[q][i] = live[q][i] ? apply_step<OPT>(a.s, pf[q][i], dl[q][i]) : pf[q][i];
            if constexpr (FULL) {
                store4<DT>(a.p, e, pf[q]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < n) store1<DT>(a.p, e + i, pf[q][i]);
            }
        }
    }

    // ---- states: new absmax and codes (8-bit) or fp32 values
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const int64_t eo = Slot<OPT>::elem_off(k, n);
        if constexpr (QUANT) {
            uint32_t w[NQ];
            float A[BPT];
            encode_tile<BS, FAST>(slot ? M2 : M1, st[k], w, A);
            float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
            uint8_t* cp = reinterpret_cast<uint8_t*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int b = 0; b < BPT; ++b)
                if (write[b] && lane == 0) am[blk0 + b] = A[b];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (write[q / QPB]) store_code_word<FULL>(cp, L::elem(base, lane, q), n, w[q]);
        } else {
            float* fp = reinterpret_cast<float*>(slot ? a.s2 : a.s1) + eo;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (!write[q / QPB]) continue;
                const int64_t e = L::elem(base, lane, q);
                if constexpr (FULL) {
                    const f32x4 v = {st[k][q][0], st[k][q][1], st[k][q][2], st[k][q][3]};
                    st_stream(v, reinterpret_cast<f32x4*>(fp + e));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (e + i < n) fp[e + i] = st[k][q][i];
                }
            }
        }
    }
}

// Index of this wave in the grid, as a scalar (wave-uniform) value.
__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// The tiles of one wave: t = first, first + stride, ...  Each tile issues all of
// its loads before any use; latency is hidden by the other waves of the CU (the
// tile code needs few enough registers for five waves per SIMD, which streams
// better here than a two-deep software pipeline at two waves per SIMD).  Tiles in
// range on aligned buffers take the vector path, the ragged last tile (or every
// tile of an unaligned call) the guarded path.
template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM, bool FAST>
__device__ __forceinline__ void step_tiles(const StepArgs& a0, const MapLDS& M1, const MapLDS& M2,
                                           const int64_t* T0) {
    using R = TileRaw<DT, OPT, BS, QUANT>;
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = a0.table ? a0.total_tiles : (a0.n + TE - 1) / TE;
    for (int64_t gt = wave_id(); gt < ntiles; gt += stride) {
        StepArgs a = a0;
        int64_t t = gt;
        if (a0.table) {
            // the tensor holding global tile gt: the last one whose first tile is <= gt
            int lo = 0, hi = a0.ntab - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (T0[mid] <= gt) lo = mid; else hi = mid - 1;
            }
            const TensorDesc& d = a0.table[__builtin_amdgcn_readfirstlane(lo)];
            a.p = d.p; a.g = d.g; a.s1 = d.s1; a.s2 = d.s2; a.a1 = d.a1; a.a2 = d.a2;
            a.n = d.n; a.nb = d.nb; a.vec = d.vec;
            t = gt - d.tile0;
        }
        R x;
        if (a.vec && (t + 1) * TE <= a.n) {
            load_tile<DT, OPT, BS, QUANT, true>(a, t * TE, lane, x);
            process_tile<DT, OPT, BS, QUANT, SKIP, UNORM, FAST, true>(a, M1, M2, t * TE, lane, x);
        } else {
            load_tile<DT, OPT, BS, QUANT, false>(a, t * TE, lane, x);
            process_tile<DT, OPT, BS, QUANT, SKIP, UNORM, FAST, false>(a, M1, M2, t * TE, lane, x);
        }
    }
}

template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM>
__global__ __launch_bounds__(kThreads) void k_step(StepArgs a) {
    constexpr int NMAPS = (OPT == kAdam || OPT == kAdemamix) ? 2 : 1;
    __shared__ float Q1[256], Q2[256], T1[256], T2[256];
    __shared__ __attribute__((aligned(16))) uint8_t B1[search::kNB];
    __shared__ __attribute__((aligned(16))) uint8_t B2[search::kNB];
    __shared__ int64_t T0[kMaxTableTensors];
    const MapLDS M1{Q1, T1, B1}, M2{Q2, T2, B2};
    if (a.table) {
        for (int i = threadIdx.x; i < a.ntab; i += kThreads) T0[i] = a.table[i].tile0;
        __syncthreads();
    }
    if constexpr (QUANT) {
        if (stage_maps<NMAPS>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2))
            step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, true>(a, M1, M2, T0);
        else
            step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, false>(a, M1, M2, T0);
    } else {
        step_tiles<DT, OPT, BS, QUANT, SKIP, UNORM, false>(a, M1, M2, T0);
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
    float A[L::BPT];
    encode_tile<BS, FAST>(M, v, w, A);
#pragma unroll
    for (int b = 0; b < L::BPT; ++b)
        if ((FULL || blk0 + b < a.nb) && lane == 0) a.absmax[blk0 + b] = A[b];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        if (FULL || blk0 + q / L::QPB < a.nb) store_code_word<FULL>(a.codes, L::elem(base, lane, q), n, w[q]);
}

template <int DT, int BS, bool FAST>
__device__ __forceinline__ void quant_tiles(const CodecArgs& a, const MapLDS& M) {
    constexpr int64_t TE = Layout<BS>::TE;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + TE - 1) / TE;
    for (int64_t t = wave_id(); t < ntiles; t += nwaves) {
        const int64_t base = t * TE;
        if (a.vec && base + TE <= a.n) quant_tile<DT, BS, FAST, true>(a, M, base, lane);
        else quant_tile<DT, BS, FAST, false>(a, M, base, lane);
    }
}

template <int DT, int BS>
__global__ __launch_bounds__(kThreads) void k_quantize(CodecArgs a) {
    __shared__ float Q[256], T[256];
    __shared__ __attribute__((aligned(16))) uint8_t B[search::kNB];
    const MapLDS M{Q, T, B};
    if (stage_maps<1>(a.qmap, nullptr, Q, nullptr, T, nullptr, B, nullptr)) quant_tiles<DT, BS, true>(a, M);
    else quant_tiles<DT, BS, false>(a, M);
}

// out[i] = qmap[codes[i]] * absmax[i / BS]; each thread handles 4 elements.
template <int DT, int BS>
__global__ __launch_bounds__(kThreads) void k_dequantize(CodecArgs a) {
    __shared__ float Q[256];
    Q[threadIdx.x] = a.qmap[threadIdx.x];
    __syncthreads();
    const int64_t nquads = (a.n + 3) / 4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t qd = (int64_t)blockIdx.x * kThreads + threadIdx.x; qd < nquads; qd += stride) {
        const int64_t e = qd * 4;
        const float A = a.absmax[e / BS];             // 4 | BS: one block per quad
        float v[4];
        if (a.vec && e + 4 <= a.n) {
            const uint32_t w = ld_stream(reinterpret_cast<const uint32_t*>(a.codes + e));
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = Q[(w >> (8 * i)) & 0xffu] * A;
            store4<DT>(a.out, e, v);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < a.n) store1<DT>(a.out, e + i, Q[a.codes[e + i]] * A);
        }
    }
}

}  // namespace bitopt
