// kernels.h -- gfx950 device code of libbitopt: the fused 8-bit block-wise
// optimizer step, its 32-bit (identity codec) twin and the block-wise codec.
//
// Work decomposition (CDNA4, wave64).  A wavefront owns a tile of CH chunks of 256
// contiguous elements; in chunk c, lane l holds elements 4l..4l+3, so every
// load/store instruction of the wave covers one contiguous 256-element span
// (16 B/lane for fp32, 8 B/lane for 16-bit, 4 B/lane of codes).  A quantization
// block is BS/256 chunks of one tile, so its absmax is an in-lane max over its
// chunks followed by one wave reduction (DPP row shifts, row broadcasts, readlane)
// with no LDS traffic and no barrier.  The 256-entry codebooks sit in LDS;
// decoding is one LDS gather, encoding a branch-free binary search plus one
// neighbour comparison.
//
// Arithmetic.  Each element operation is one IEEE fp32 operation in a fixed order
// (the build disables FMA contraction and keeps correctly rounded division and
// square root), so results do not depend on the tiling and are reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

template <int OPT> struct NumStates { static constexpr int v = OPT == kAdemamix ? 3 : (OPT == kAdam ? 2 : 1); };

// ---------------------------------------------------------------- number formats

template <int DT> struct Elem;
template <> struct Elem<kF32>  { using T = float;    using Raw4 = uint4; };
template <> struct Elem<kF16>  { using T = uint16_t; using Raw4 = uint2; };
template <> struct Elem<kBF16> { using T = uint16_t; using Raw4 = uint2; };

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_half_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32, round to nearest even
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;   // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                               // nearest even
    return u >> 16;
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
    const Raw4 r = *reinterpret_cast<const Raw4*>(reinterpret_cast<const typename Elem<DT>::T*>(base) + e);
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
        r.x = narrow<DT>(v[0]) | (narrow<DT>(v[1]) << 16);
        r.y = narrow<DT>(v[2]) | (narrow<DT>(v[3]) << 16);
    }
    *reinterpret_cast<Raw4*>(reinterpret_cast<typename Elem<DT>::T*>(base) + e) = r;
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

// ---------------------------------------------------------------- fused step tile

// One wave processes one tile: CH chunks of 256 elements starting at `base`.
// QUANT: 8-bit block-wise states (codes + absmax); otherwise fp32 states.
// FULL: the whole tile is in range and every buffer aligned (vector path).
template <int DT, int OPT, int BS, int CH, bool QUANT, bool SKIP, bool UNORM, bool FULL>
__device__ __forceinline__ void step_tile(const StepArgs& a, const float* Q1, const float* Q2,
                                          int64_t base, int lane) {
    constexpr int NS = NumStates<OPT>::v;
    constexpr int CPB = BS / 256;          // chunks per block
    constexpr int BPT = CH / CPB;          // blocks per tile
    static_assert(CH % CPB == 0, "a tile holds whole blocks");
    const int64_t n = a.n;
    const int64_t blk0 = base / BS;

    float pf[CH][4], gf[CH][4], st[NS][CH][4];
    bool live[CH][4];

    // ---- loads (all issued before any use) and decode
    uint32_t code[NS][CH];
    float4 fst[NS][CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = base + c * 256 + lane * 4;
        if constexpr (FULL) {
            load4<DT>(a.p, e, pf[c]);
            load4<DT>(a.g, e, gf[c]);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int slot = Slot<OPT>::which(k);
                const int64_t eo = Slot<OPT>::elem_off(k, n) + e;
                if constexpr (QUANT) code[k][c] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + eo);
                else fst[k][c] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(slot ? a.s2 : a.s1) + eo);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = e + i < n;
                pf[c][i] = ok ? load1<DT>(a.p, e + i) : 0.0f;
                gf[c][i] = ok ? load1<DT>(a.g, e + i) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int slot = Slot<OPT>::which(k);
                const int64_t eo = Slot<OPT>::elem_off(k, n) + e;
                if constexpr (QUANT) {
                    const uint8_t* cp = reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + eo;
                    uint32_t w = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w |= (e + i < n ? (uint32_t)cp[i] : 0u) << (8 * i);
                    code[k][c] = w;
                } else {
                    const float* fp = reinterpret_cast<const float*>(slot ? a.s2 : a.s1) + eo;
                    fst[k][c].x = e + 0 < n ? fp[0] : 0.0f;
                    fst[k][c].y = e + 1 < n ? fp[1] : 0.0f;
                    fst[k][c].z = e + 2 < n ? fp[2] : 0.0f;
                    fst[k][c].w = e + 3 < n ? fp[3] : 0.0f;
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const float* Q = slot ? Q2 : Q1;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t e = base + c * 256 + lane * 4;
            if constexpr (QUANT) {
                const int64_t b = blk0 + c / CPB;
                const float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
                const float A = (FULL || b < a.nb) ? am[b] : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = Q[(code[k][c] >> (8 * i)) & 0xffu] * A;
                    st[k][c][i] = (FULL || e + i < n) ? v : 0.0f;
                }
            } else {
                st[k][c][0] = fst[k][c].x; st[k][c][1] = fst[k][c].y;
                st[k][c][2] = fst[k][c].z; st[k][c][3] = fst[k][c].w;
            }
        }
    }

    // ---- element updates
    float dl[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = base + c * 256 + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = FULL || (e + i < n);
            const bool skip = SKIP && (gf[c][i] == 0.0f);   // raw gradient; -0 counts as zero
            live[c][i] = valid && !skip;
            float s3[3] = {st[0][c][i], NS > 1 ? st[NS > 1 ? 1 : 0][c][i] : 0.0f,
                           NS > 2 ? st[NS > 2 ? 2 : 0][c][i] : 0.0f};
            float d;
            update_elem<OPT>(a.s, pf[c][i], gf[c][i], s3, d);
            dl[c][i] = live[c][i] ? d : 0.0f;
#pragma unroll
            for (int k = 0; k < NS; ++k) st[k][c][i] = live[c][i] ? s3[k] : st[k][c][i];
        }
    }

    // ---- per-block cap of the update norm
    if constexpr (UNORM) {
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            double su = 0.0, sp = 0.0;
#pragma unroll
            for (int cc = 0; cc < CPB; ++cc) {
                const int c = j * CPB + cc;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d2 = dl[c][i] * dl[c][i];
                    const float p2 = pf[c][i] * pf[c][i];
                    su += (double)d2;
                    sp += (double)p2;
                }
            }
            su = wave_sum_f64(su);
            sp = wave_sum_f64(sp);
            const double U = sqrt(su), P = sqrt(sp);
            const double lim = (double)a.s.max_unorm * P;
            if (U > lim) {
                const float clip = (float)(lim / U);
#pragma unroll
                for (int cc = 0; cc < CPB; ++cc) {
                    const int c = j * CPB + cc;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dl[c][i] = dl[c][i] * clip;
                }
            }
        }
    }

    // ---- new parameters (skipped and invalid elements keep theirs)
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pn = apply_step<OPT>(a.s, pf[c][i], dl[c][i]);
            pf[c][i] = live[c][i] ? pn : pf[c][i];
        }

    // ---- per block: skip test, new absmax, encode, stores
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int64_t b = blk0 + j;
        if (!FULL && b >= a.nb) break;                 // wave-uniform
        if constexpr (SKIP) {
            bool any = false;
#pragma unroll
            for (int cc = 0; cc < CPB; ++cc)
#pragma unroll
                for (int i = 0; i < 4; ++i) any = any || live[j * CPB + cc][i];
            if (!wave_any(any)) continue;              // every gradient zero: block untouched
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int slot = Slot<OPT>::which(k);
            if constexpr (QUANT) {
                const float* Q = slot ? Q2 : Q1;
                float m = 0.0f;
#pragma unroll
                for (int cc = 0; cc < CPB; ++cc)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(st[k][j * CPB + cc][i]));
                const float A = wave_max_nonneg(m);
                const float r = (A == 0.0f) ? 0.0f : 1.0f / A;
                float* am = (slot ? a.a2 : a.a1) + Slot<OPT>::block_off(k, a.nb);
                if (lane == 0) am[b] = A;
                uint8_t* cp = reinterpret_cast<uint8_t*>(slot ? a.s2 : a.s1) + Slot<OPT>::elem_off(k, n);
#pragma unroll
                for (int cc = 0; cc < CPB; ++cc) {
                    const int c = j * CPB + cc;
                    const int64_t e = base + c * 256 + lane * 4;
                    uint32_t w = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = st[k][c][i] * r;
                        w |= nearest_code(Q, x) << (8 * i);
                    }
                    if constexpr (FULL) {
                        *reinterpret_cast<uint32_t*>(cp + e) = w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (e + i < n) cp[e + i] = (uint8_t)(w >> (8 * i));
                    }
                }
            } else {
                float* fp = reinterpret_cast<float*>(slot ? a.s2 : a.s1) + Slot<OPT>::elem_off(k, n);
#pragma unroll
                for (int cc = 0; cc < CPB; ++cc) {
                    const int c = j * CPB + cc;
                    const int64_t e = base + c * 256 + lane * 4;
                    if constexpr (FULL) {
                        *reinterpret_cast<float4*>(fp + e) = make_float4(st[k][c][0], st[k][c][1], st[k][c][2], st[k][c][3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (e + i < n) fp[e + i] = st[k][c][i];
                    }
                }
            }
        }
#pragma unroll
        for (int cc = 0; cc < CPB; ++cc) {
            const int c = j * CPB + cc;
            const int64_t e = base + c * 256 + lane * 4;
            if constexpr (FULL) {
                store4<DT>(a.p, e, pf[c]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < n) store1<DT>(a.p, e + i, pf[c][i]);
            }
        }
    }
}

template <int BS> struct TileChunks { static constexpr int v = BS >= 1024 ? BS / 256 : 4; };

template <int DT, int OPT, int BS, bool QUANT, bool SKIP, bool UNORM>
__global__ __launch_bounds__(kThreads) void k_step(StepArgs a) {
    constexpr int CH = TileChunks<BS>::v;
    constexpr int64_t TE = (int64_t)CH * 256;
    __shared__ float Q1[256];
    __shared__ float Q2[256];
    if constexpr (QUANT) {
        Q1[threadIdx.x] = a.q1[threadIdx.x];
        if constexpr (OPT == kAdam || OPT == kAdemamix) Q2[threadIdx.x] = a.q2[threadIdx.x];
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + TE - 1) / TE;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6); t < ntiles; t += nwaves) {
        const int64_t base = t * TE;
        if (a.vec && base + TE <= a.n)
            step_tile<DT, OPT, BS, CH, QUANT, SKIP, UNORM, true>(a, Q1, Q2, base, lane);
        else
            step_tile<DT, OPT, BS, CH, QUANT, SKIP, UNORM, false>(a, Q1, Q2, base, lane);
    }
}

// ---------------------------------------------------------------- codec kernels

struct CodecArgs {
    const void* x;       // quantize input / dequantize output
    void* out;
    uint8_t* codes;
    float* absmax;
    const float* qmap;
    int64_t n;
    int64_t nb;
    int32_t vec;
};

template <int DT, int BS, bool FULL>
__device__ __forceinline__ void quant_tile(const CodecArgs& a, const float* Q, int64_t base, int lane) {
    constexpr int CH = TileChunks<BS>::v;
    constexpr int CPB = BS / 256;
    constexpr int BPT = CH / CPB;
    const int64_t n = a.n;
    float v[CH][4];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = base + c * 256 + lane * 4;
        if constexpr (FULL) load4<DT>(a.x, e, v[c]);
        else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[c][i] = e + i < n ? load1<DT>(a.x, e + i) : 0.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int64_t b = base / BS + j;
        if (!FULL && b >= a.nb) break;
        float m = 0.0f;
#pragma unroll
        for (int cc = 0; cc < CPB; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(v[j * CPB + cc][i]));
        const float A = wave_max_nonneg(m);
        const float r = (A == 0.0f) ? 0.0f : 1.0f / A;
        if (lane == 0) a.absmax[b] = A;
#pragma unroll
        for (int cc = 0; cc < CPB; ++cc) {
            const int c = j * CPB + cc;
            const int64_t e = base + c * 256 + lane * 4;
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = v[c][i] * r;
                w |= nearest_code(Q, x) << (8 * i);
            }
            if constexpr (FULL) *reinterpret_cast<uint32_t*>(a.codes + e) = w;
            else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < n) a.codes[e + i] = (uint8_t)(w >> (8 * i));
            }
        }
    }
}

template <int DT, int BS>
__global__ __launch_bounds__(kThreads) void k_quantize(CodecArgs a) {
    constexpr int64_t TE = (int64_t)TileChunks<BS>::v * 256;
    __shared__ float Q[256];
    Q[threadIdx.x] = a.qmap[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + TE - 1) / TE;
    for (int64_t t = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6); t < ntiles; t += nwaves) {
        const int64_t base = t * TE;
        if (a.vec && base + TE <= a.n) quant_tile<DT, BS, true>(a, Q, base, lane);
        else quant_tile<DT, BS, false>(a, Q, base, lane);
    }
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
            const uint32_t w = *reinterpret_cast<const uint32_t*>(a.codes + e);
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
