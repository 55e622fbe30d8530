// tensorwise.h -- the non-block-wise (tensor-wide) 8-bit step: every state has one
// absmax for the whole tensor.  The new absmax depends on every element's new state,
// so the step takes three launches:
//   pass 1   reads g, the codes and (where the state update uses it) p, computes the
//            new states, and each group writes its max |state| per state (and whether
//            it saw a nonzero gradient) to its own workspace slot -- no atomics, so
//            no contention on a few addresses and a deterministic result;
//   reduce   one group folds the slots into the tensor-wide absmax and copies the
//            old absmax next to it (pass 2 decodes with the copy, so it may
//            overwrite the absmax array);
//   pass 2   reads everything again, recomputes the same values, writes p, encodes
//            the states with the tensor-wide scale and writes the codes and absmax.
// With max_unorm (UNORM), pass 1 also reads p and sums the squares of the update and
// of the parameters (fp32 squares, double sums), the reduction turns the two sums
// into the tensor's clip factor, and pass 2 scales every update by it.
// Workspace words: [0, 3) new absmax bits per state, [3, 6) old absmax, [6] nonzero
// gradient seen, [7] clip factor (1 when the norm is within the cap); then
// kTwWordsPerPart words per group of pass 1: the max bits of up to three states, the
// nonzero-gradient flag and the two sums as double bit patterns split into word
// pairs (a maximum of non-negative floats is taken on their bit patterns as integers).
// The element arithmetic is update_elem / apply_step / encode of kernels.h, so the
// results equal one block spanning the tensor.
#pragma once

#include "kernels.h"

namespace bitopt {

constexpr int kTwHead = 8;                 // words before the per-group slots
constexpr int kTwWordsPerPart = 8;         // 3 max bits, nonzero-gradient flag, 2 x double sum
constexpr int kTwMaxParts = 1024;          // groups of pass 1 (grid-stride beyond)
constexpr int kTwWords = kTwHead + kTwWordsPerPart * kTwMaxParts;

// One quad of lane l of a tile: element indices e .. e+3 (FULL: in range and aligned).
template <int DT, int OPT, bool SKIP, bool FULL, bool NEEDP>
__device__ __forceinline__ void tw_quad(const StepArgs& a, const float* const (&Q)[2], const float (&A)[3],
                                        int64_t e, float (&pv)[4], float (&st)[3][4], float (&dl)[4],
                                        uint32_t& livem) {
    constexpr int NS = NumStates<OPT>::v;
    const int64_t n = a.n;
    float gv[4];
    if constexpr (FULL) {
        if constexpr (NEEDP) load4<DT>(a.p, e, pv);
        else pv[0] = pv[1] = pv[2] = pv[3] = 0.0f;
        load4<DT>(a.g, e, gv);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = e + i < n;
            pv[i] = (NEEDP && valid) ? load1<DT>(a.p, e + i) : 0.0f;
            gv[i] = valid ? load1<DT>(a.g, e + i) : 0.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = Slot<OPT>::which(k);
        const uint8_t* cp = reinterpret_cast<const uint8_t*>(slot ? a.s2 : a.s1) + Slot<OPT>::elem_off(k, n);
        if constexpr (FULL) {
            const uint32_t w = ld_stream(reinterpret_cast<const uint32_t*>(cp + e));
#pragma unroll
            for (int i = 0; i < 4; ++i) st[k][i] = Q[slot][(w >> (8 * i)) & 0xffu] * A[k];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) st[k][i] = e + i < n ? Q[slot][gbl(cp)[e + i]] * A[k] : 0.0f;
        }
    }
    livem = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool valid = FULL || e + i < n;
        const bool live = valid && !(SKIP && gv[i] == 0.0f);
        livem |= live ? 1u << i : 0u;
        float s3[3] = {st[0][i], NS > 1 ? st[NS > 1 ? 1 : 0][i] : 0.0f, NS > 2 ? st[NS > 2 ? 2 : 0][i] : 0.0f};
        float d;
        update_elem<OPT>(a.s, pv[i], gv[i], s3, d);
        dl[i] = live ? d : 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) st[k][i] = live ? s3[k] : st[k][i];
    }
}

template <int OPT>
__device__ __forceinline__ void tw_old_absmax(const StepArgs& a, float (&A)[3]) {
#pragma unroll
    for (int k = 0; k < 3; ++k) A[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < NumStates<OPT>::v; ++k) {
        const float* am = (Slot<OPT>::which(k) ? a.a2 : a.a1) + Slot<OPT>::block_off(k, 1);
        A[k] = gbl(am)[0];
    }
}

__device__ __forceinline__ void tw_put_f64(uint32_t* w, double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    w[0] = (uint32_t)b;
    w[1] = (uint32_t)(b >> 32);
}
__device__ __forceinline__ double tw_get_f64(const uint32_t* w) {
    return __longlong_as_double((long long)(((uint64_t)w[1] << 32) | w[0]));
}

// Pass 1: the tensor-wide max |new state| of each state (UNORM: and the sums of
// squares of the update and of the parameters).
template <int DT, int OPT, bool SKIP, bool UNORM>
__global__ __launch_bounds__(kThreads) void k_tw_max(StepArgs a) {
    constexpr int NS = NumStates<OPT>::v;
    constexpr bool NEEDP = StateReadsP<OPT>::v || UNORM;
    constexpr int NMAPS = (OPT == kAdam || OPT == kAdemamix) ? 2 : 1;
    __shared__ float Q1[256], Q2[256];
    Q1[threadIdx.x] = gbl(a.q1)[threadIdx.x];
    if constexpr (NMAPS > 1) Q2[threadIdx.x] = gbl(a.q2)[threadIdx.x];
    __syncthreads();
    const float* const Q[2] = {Q1, Q2};
    float A[3];
    tw_old_absmax<OPT>(a, A);

    const int lane = threadIdx.x & 63;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + 1023) / 1024;
    float mx[3] = {0.0f, 0.0f, 0.0f};
    uint32_t anyl = 0;
    double su = 0.0, sp = 0.0;
    for (int64_t t = wave_id(); t < ntiles; t += stride) {
        const bool full = a.vec && (t + 1) * 1024 <= a.n;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t e = t * 1024 + q * 256 + lane * 4;
            float pv[4], st[3][4], dl[4];
            uint32_t livem;
            if (full) tw_quad<DT, OPT, SKIP, true, NEEDP>(a, Q, A, e, pv, st, dl, livem);
            else tw_quad<DT, OPT, SKIP, false, NEEDP>(a, Q, A, e, pv, st, dl, livem);
            anyl |= livem;
#pragma unroll
            for (int k = 0; k < NS; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx[k] = fmaxf(mx[k], fabsf(st[k][i]));
            if constexpr (UNORM) {
                // skipped and out-of-range elements have a zero update, and
                // out-of-range ones a zero parameter: they add nothing
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d2 = dl[i] * dl[i];
                    const float p2 = pv[i] * pv[i];
                    su += (double)d2;
                    sp += (double)p2;
                }
            }
        }
    }
    // this group's slot: per-wave results through LDS, one lane writes
    __shared__ uint32_t part[kWavesPerGroup][4];
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float m = k < NS ? wave_max_nonneg(mx[k]) : 0.0f;
        if (lane == 0) part[wave][k] = __float_as_uint(m);
    }
    const bool any = wave_any(anyl != 0u);
    if (lane == 0) part[wave][3] = any ? 1u : 0u;
    __shared__ double sums[kWavesPerGroup][2];
    if constexpr (UNORM) {
        su = wave_sum_f64(su);
        sp = wave_sum_f64(sp);
        if (lane == 0) { sums[wave][0] = su; sums[wave][1] = sp; }
    }
    __syncthreads();
    uint32_t* slot = a.ws + kTwHead + kTwWordsPerPart * blockIdx.x;
    if (threadIdx.x < 4) {
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) v = max(v, part[w][threadIdx.x]);
        slot[threadIdx.x] = v;
    } else if (threadIdx.x < 6) {
        const int j = threadIdx.x - 4;
        double v = 0.0;
        if constexpr (UNORM) {
#pragma unroll
            for (int w = 0; w < kWavesPerGroup; ++w) v += sums[w][j];
        }
        tw_put_f64(slot + 4 + 2 * j, v);
    }
}

// Fold the pass-1 slots into the tensor-wide results; copy the old absmax.  UNORM:
// the clip factor, max_unorm * P / U when U > max_unorm * P (U, P: the norms of the
// update and of the parameters), else 1.  The sums are folded in a fixed order, so
// the result does not depend on timing.
template <int OPT, bool UNORM>
__global__ __launch_bounds__(kThreads) void k_tw_reduce(StepArgs a) {
    constexpr int NS = NumStates<OPT>::v;
    __shared__ uint32_t red[kWavesPerGroup][4];
    __shared__ double sums[kWavesPerGroup][2];
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    double su = 0.0, sp = 0.0;
    for (int i = threadIdx.x; i < a.parts; i += kThreads) {
        const uint32_t* slot = a.ws + kTwHead + kTwWordsPerPart * i;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = max(v[j], slot[j]);
        if constexpr (UNORM) {
            su += tw_get_f64(slot + 4);
            sp += tw_get_f64(slot + 6);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = __float_as_uint(wave_max_nonneg(__uint_as_float(v[j])));
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6][j] = w;
    }
    if constexpr (UNORM) {
        su = wave_sum_f64(su);
        sp = wave_sum_f64(sp);
        if ((threadIdx.x & 63) == 0) { sums[threadIdx.x >> 6][0] = su; sums[threadIdx.x >> 6][1] = sp; }
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) r = max(r, red[w][threadIdx.x]);
        a.ws[threadIdx.x < 3 ? threadIdx.x : 6] = r;
    }
    if (threadIdx.x == 4) {
        float clip = 1.0f;
        if constexpr (UNORM) {
            double tu = 0.0, tp = 0.0;
#pragma unroll
            for (int w = 0; w < kWavesPerGroup; ++w) { tu += sums[w][0]; tp += sums[w][1]; }
            const double U = sqrt(tu), P = sqrt(tp);
            const double lim = (double)a.s.max_unorm * P;
            if (U > lim) clip = (float)(lim / U);
        }
        a.ws[7] = __float_as_uint(clip);
    }
    if (threadIdx.x < NS) {
        float A[3];
        tw_old_absmax<OPT>(a, A);
        a.ws[3 + threadIdx.x] = __float_as_uint(A[threadIdx.x]);
    }
}

// Pass 2: recompute, write p, encode with the tensor-wide scale, write codes and absmax.
template <int DT, int OPT, bool SKIP, bool UNORM>
__global__ __launch_bounds__(kThreads) void k_tw_apply(StepArgs a) {
    constexpr int NS = NumStates<OPT>::v;
    constexpr int NMAPS = (OPT == kAdam || OPT == kAdemamix) ? 2 : 1;
    if (SKIP && a.ws[6] == 0u) return;                 // no nonzero gradient: nothing is written
    __shared__ float Q1[256], Q2[256], T1[256], T2[256];
    __shared__ __attribute__((aligned(16))) uint8_t B1[search::kNB];
    __shared__ __attribute__((aligned(16))) uint8_t B2[search::kNB];
    __shared__ uint32_t vote[kWavesPerGroup];
    const bool fast = stage_maps<NMAPS, UnsignedState1<OPT>::v>(a.q1, a.q2, Q1, Q2, T1, T2, B1, B2, vote);
    const MapLDS M[2] = {MapLDS{Q1, T1, B1}, MapLDS{Q2, T2, B2}};
    const float* const Q[2] = {Q1, Q2};
    float A[3], r[3], c[3], rs[3];
    bool tab[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        A[k] = k < NS ? __uint_as_float(a.ws[3 + k]) : 0.0f;
        const float An = k < NS ? __uint_as_float(a.ws[k]) : 0.0f;
        block_recip(An, r[k], c[k]);
        tab[k] = fast && table_recip_ok(r[k]);
        rs[k] = r[k] * kEncScale;
    }
    const float clip = UNORM ? __uint_as_float(a.ws[7]) : 1.0f;
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x < NS) {
        const int k = threadIdx.x;
        float* am = (Slot<OPT>::which(k) ? a.a2 : a.a1) + Slot<OPT>::block_off(k, 1);
        gbl(am)[0] = __uint_as_float(a.ws[k]);
    }
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    const int64_t ntiles = (a.n + 1023) / 1024;
    for (int64_t t = wave_id(); t < ntiles; t += stride) {
        const bool full = a.vec && (t + 1) * 1024 <= a.n;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t e = t * 1024 + q * 256 + lane * 4;
            float pv[4], st[3][4], dl[4];
            uint32_t livem;
            if (full) tw_quad<DT, OPT, SKIP, true, true>(a, Q, A, e, pv, st, dl, livem);
            else tw_quad<DT, OPT, SKIP, false, true>(a, Q, A, e, pv, st, dl, livem);
            if constexpr (UNORM) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dl[i] = dl[i] * clip;   // x * 1 == x: no clip, same bits
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = ((livem >> i) & 1u) ? apply_step<OPT>(a.s, pv[i], dl[i]) : pv[i];
            if (full) {
                store4<DT>(a.p, e, pv);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (e + i < a.n) store1<DT>(a.p, e + i, pv[i]);
            }
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int slot = Slot<OPT>::which(k);
                uint32_t w = 0;
                if (tab[k]) {                                       // uniform
#pragma unroll
                    for (int i = 0; i < 4; ++i) w |= encode<true>(M[slot], (st[k][i] * c[k]) * rs[k]) << (8 * i);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) w |= encode<false>(M[slot], (st[k][i] * c[k]) * r[k]) << (8 * i);
                }
                uint8_t* cp = reinterpret_cast<uint8_t*>(slot ? a.s2 : a.s1) + Slot<OPT>::elem_off(k, a.n);
                if (full) store_code_word<true>(cp, e, a.n, w);
                else store_code_word<false>(cp, e, a.n, w);
            }
        }
    }
}

}  // namespace bitopt
