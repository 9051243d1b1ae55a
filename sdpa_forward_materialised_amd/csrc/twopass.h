// Two-sweep kernel: row statistics, then probabilities and output.
//
// Math (FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton +
// P800 exact-P/A1)", "P800 exact-P fast path" update): once the row-wise
// log-sum-exp is known, P = exp(scale * Q K^T - LSE) is exact. Sweep 1 over
// the keys finds the row maximum and sum (online, base 2) and so LSE; sweep 2
// recomputes each score tile, writes P = exp2(t - lse2) rounded to the
// output dtype, and accumulates O^T += V^T P^T from exactly those rounded
// values. Scores live in the base-2 domain with scale * log2(e) folded into
// one multiplier (as the cudnn-frontend merge-log notes do for their
// kernels). Unlike the page's two-stage Triton path, P is never read back:
// P·V is accumulated in the pass that writes it.
//
// One workgroup = NW waves x 32 query rows of one (batch, query head). Each
// 64-key tile of K (both sweeps) and V^T (sweep 2) is staged through LDS once
// and shared by all waves; tiles are double-buffered with the next one
// prefetched into registers while the current one is consumed, so one
// barrier per tile suffices. Every global access goes through a buffer
// descriptor with out-of-range lanes predicated off (no branches), all loads
// a tile needs are issued before the previous tile's probability stores, and
// the causal zero region is written after the last tile.

#pragma once

#include "sdpa_device.h"

namespace sdpa {

// Mask bits for the 64 keys of one tile, fetched one tile ahead.
template <typename T, int MASK, bool VEC>
struct MaskPrefetch {
    __device__ __forceinline__ void load(const FwdArgs&, rsrc_t, uint32_t, int, int) {}
    __device__ __forceinline__ void get(const FwdArgs&, rsrc_t, uint32_t, int, int, int, float*) const {}
};

// Vectorised masks: per lane 4 runs of 8 keys (2 blocks x 2 runs).
template <typename T, int MASK>
struct MaskPrefetch<T, MASK, true> {
    static constexpr int ME = MASK == MASK_BOOL ? 1 : (int)sizeof(T);
    static constexpr int NCH = MASK == MASK_NONE ? 0 : (ME == 4 ? 8 : 4);  // 16-byte chunks (bool: 8 bytes)
    u32x4 raw[NCH > 0 ? NCH : 1];

    __device__ __forceinline__ void load(const FwdArgs& a, rsrc_t mr, uint32_t row_off, int k0, int hf) {
        if constexpr (MASK != MASK_NONE) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = k0 + 32 * (q >> 1) + 16 * (q & 1) + 8 * hf;
                const uint32_t off = pred(j < a.Skv, row_off + (uint32_t)j * ME);
                if constexpr (ME == 1) {
                    const u32x2 w = ld64(mr, off);
                    raw[q] = u32x4{w[0], w[1], 0u, 0u};
                } else if constexpr (ME == 2) {
                    raw[q] = ld128(mr, off);
                } else {
                    raw[2 * q] = ld128(mr, off);
                    raw[2 * q + 1] = ld128(mr, off == OOB ? OOB : off + 16);
                }
            }
        }
    }
    // decoded terms for block kb (16 values in accumulator-register order)
    __device__ __forceinline__ void get(const FwdArgs&, rsrc_t, uint32_t, int, int, int kb, float* out) const {
        if constexpr (MASK != MASK_NONE) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int q = 2 * kb + c;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v;
                    if constexpr (MASK == MASK_BOOL) {
                        v = ((raw[q][e >> 2] >> (8 * (e & 3))) & 0xffu) ? 1.0f : 0.0f;
                    } else if constexpr (ME == 2) {
                        v = Tr<T>::to_f((raw[q][e >> 1] >> (16 * (e & 1))) & 0xffffu) * LOG2E;
                    } else {
                        v = __builtin_bit_cast(float, raw[2 * q + (e >> 2)][e & 3]) * LOG2E;
                    }
                    out[8 * c + e] = v;
                }
            }
        }
    }
};

// Element-wise masks (any layout): read when needed.
template <typename T, int MASK>
struct MaskPrefetch<T, MASK, false> {
    __device__ __forceinline__ void load(const FwdArgs&, rsrc_t, uint32_t, int, int) {}
    __device__ __forceinline__ void get(const FwdArgs& a, rsrc_t mr, uint32_t row_off, int k0, int hf, int kb,
                                        float* out) const {
        if constexpr (MASK != MASK_NONE) load_mask16<T, MASK, false>(a, mr, row_off, k0 + 32 * kb, hf, out);
    }
};

template <typename T, int D, int NW, int MASK, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2)))
void sdpa_twopass_kernel(const FwdArgs a) {
    using TR = Tr<T>;
    using vec = typename TR::vec;
    constexpr int SZ = (int)sizeof(T);
    constexpr int KH = TR::KH;
    constexpr int KSTEP = 2 * KH;
    constexpr int NKS = D / KSTEP;           // MFMAs per 32x32 score block
    constexpr int NT = NW * 64;
    constexpr int QB = 32 * NW;
    constexpr int E16 = 16 / SZ;             // elements per 16-byte chunk
    constexpr int KLD = D + E16;             // LDS row pitch of a K tile (padded)
    constexpr int VLD = BN + E16;            // LDS row pitch of a V^T tile (padded)
    constexpr int CPR = D / E16;             // 16-byte chunks per K/V row
    constexpr int KCH = (BN * CPR + NT - 1) / NT;        // K chunks per thread
    constexpr int NVI = (BN / 4) * CPR;                  // V items: 4 keys x one chunk
    constexpr int VIT = (NVI + NT - 1) / NT;             // V items per thread
    constexpr int ND = D / 32;               // 32-wide head-dim chunks of O^T
    constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;

    __shared__ __attribute__((aligned(16))) T k_lds[2][BN * KLD];
    __shared__ __attribute__((aligned(16))) T vt_lds[2][D * VLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int n = lane & 31;
    const int hf = lane >> 5;

    const Work w = decode_block(blockIdx.x, a);
    const int hk = w.hq / a.group;
    const int q0 = w.qblk * QB;
    const int qw = q0 + 32 * wave;
    const int qi = qw + n;
    const bool row_ok = qi < a.Sq;

    const int kend = a.causal ? min(a.Skv, q0 + QB) : a.Skv;
    const int ntiles = (kend + BN - 1) / BN;

    const rsrc_t qr = make_rsrc(static_cast<const T*>(a.q) + w.b * a.q_s[0] + w.hq * a.q_s[1], a.q_ext);
    const rsrc_t kr = make_rsrc(static_cast<const T*>(a.k) + w.b * a.k_s[0] + hk * a.k_s[1], a.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(a.v) + w.b * a.v_s[0] + hk * a.v_s[1], a.v_ext);
    const rsrc_t pr = make_rsrc(static_cast<T*>(a.p) + w.b * a.p_s[0] + w.hq * a.p_s[1], a.p_ext);
    const rsrc_t orr = make_rsrc(static_cast<T*>(a.o) + w.b * a.o_s[0] + w.hq * a.o_s[1], a.o_ext);
    const rsrc_t lr = make_rsrc(a.lse + w.b * a.l_s[0] + w.hq * a.l_s[1], a.l_ext);
    rsrc_t mr = kr;
    uint32_t mrow_off = 0;
    if constexpr (MASK != MASK_NONE) {
        mr = make_rsrc(static_cast<const uint8_t*>(a.mask) + (w.b * a.m_s[0] + w.hq * a.m_s[1]) * ME, a.m_ext);
        mrow_off = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.m_s[2] * ME);
    }
    const uint32_t prow_off = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.p_s[2] * SZ);

    // Q fragments (B operand): lane (n, h) holds Q[qi][c*KSTEP + h*KH .. +KH)
    vec qf[NKS];
    {
        const uint32_t qoff = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.q_s[2] * SZ);
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            const uint32_t off = pred(row_ok, qoff + (uint32_t)((c * KSTEP + hf * KH) * SZ));
            if constexpr (SZ == 2) qf[c] = as_vec<T>(ld128(qr, off));
            else qf[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, off, 0, 0));
        }
    }

    // ---- tile staging (registers -> LDS)
    u32x4 kreg[KCH];
    u32x4 vreg[VIT][4];
    MaskPrefetch<T, MASK, VEC> mpre;  // mask bits of the tile after the staged one

    auto load_k = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            const int row = c / CPR, ch = c - (c / CPR) * CPR;
            const bool ok = (c < BN * CPR) && (k0 + row < a.Skv);
            kreg[i] = ld128(kr, pred(ok, (uint32_t)((int64_t)(k0 + row) * a.k_s[2] * SZ) + (uint32_t)(ch * 16)));
        }
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            if (KCH * NT == BN * CPR || c < BN * CPR) {
                const int row = c / CPR, ch = c - (c / CPR) * CPR;
                *reinterpret_cast<u32x4*>(&k_lds[buf][row * KLD + ch * E16]) = kreg[i];
            }
        }
    };
    auto load_v = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
            const int it = tid + i * NT;
            const int kg = it / CPR, ch = it - (it / CPR) * CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 4 * kg + r;
                const bool ok = (VIT * NT == NVI || it < NVI) && key < a.Skv;
                vreg[i][r] = ld128(vr, pred(ok, (uint32_t)((int64_t)key * a.v_s[2] * SZ) + (uint32_t)(ch * 16)));
            }
        }
    };
    auto store_vt = [&](int buf) {
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
            const int it = tid + i * NT;
            if (VIT * NT == NVI || it < NVI) {
                const int kg = it / CPR, ch = it - (it / CPR) * CPR;
                if constexpr (SZ == 2) {
                    // 8 head-dim rows, each receiving 4 consecutive keys (8 bytes)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int wd = e >> 1;
                        const uint32_t x0 = vreg[i][0][wd], x1 = vreg[i][1][wd];
                        const uint32_t x2 = vreg[i][2][wd], x3 = vreg[i][3][wd];
                        uint32_t lo, hi;
                        if (e & 1) {
                            lo = (x0 >> 16) | (x1 & 0xffff0000u);
                            hi = (x2 >> 16) | (x3 & 0xffff0000u);
                        } else {
                            lo = (x0 & 0xffffu) | (x1 << 16);
                            hi = (x2 & 0xffffu) | (x3 << 16);
                        }
                        *reinterpret_cast<u32x2*>(&vt_lds[buf][(ch * 8 + e) * VLD + 4 * kg]) = u32x2{lo, hi};
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<u32x4*>(&vt_lds[buf][(ch * 4 + e) * VLD + 4 * kg]) =
                            u32x4{vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
                }
            }
        }
    };

    // S^T of both 32-key blocks of the staged tile for this wave's queries
    // (two independent MFMA chains, interleaved to cover their latency).
    auto qk_tile = [&](int buf, f32x16* acc) {
        acc[0] = f32x16{};
        acc[1] = f32x16{};
        const T* k0row = &k_lds[buf][swap23(n) * KLD + hf * KH];
        const T* k1row = k0row + 32 * KLD;
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            vec a0, a1;
            if constexpr (SZ == 2) {
                a0 = as_vec<T>(*reinterpret_cast<const u32x4*>(k0row + c * KSTEP));
                a1 = as_vec<T>(*reinterpret_cast<const u32x4*>(k1row + c * KSTEP));
            } else {
                a0 = k0row[c * KSTEP];
                a1 = k1row[c * KSTEP];
            }
            acc[0] = TR::mfma(a0, qf[c], acc[0]);
            acc[1] = TR::mfma(a1, qf[c], acc[1]);
        }
    };

    // ---------------- sweep 1: row maximum and sum (base 2)
    // Loop shape: compute tile t from LDS buffer t&1, then stage tile t+1
    // (already in registers) into the other buffer, barrier, and prefetch
    // tile t+2. Every path into the LDS writes then has the same memory ops
    // in flight (the prefetch, then this tile's stores), so the counter wait
    // there never covers the probability stores.
    float m_run = -INFINITY, l_run = 0.0f;
    MaskPrefetch<T, MASK, VEC> mcur;
    if (ntiles > 0) {
        load_k(0);
        mpre.load(a, mr, mrow_off, 0, hf);
        store_k(0);
        mcur = mpre;
        __syncthreads();
        const int t1 = min(1, ntiles - 1);
        load_k(t1);
        mpre.load(a, mr, mrow_off, t1 * BN, hf);
    }
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * BN;
        const int buf = t & 1;
        if (!(a.causal && k0 > qw + 31)) {  // else: whole tile above this wave's diagonal
            const bool edge = (k0 + BN > a.Skv) || (a.causal && k0 + BN - 1 > qw);
            f32x16 acc2[2];
            qk_tile(buf, acc2);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float mv[16];
                mcur.get(a, mr, mrow_off, k0, hf, kb, mv);
                float tt[16];
                if (edge) scores16<MASK>(a, acc2[kb], mv, k0 + 32 * kb, hf, qi, true, tt);
                else scores16<MASK>(a, acc2[kb], mv, k0 + 32 * kb, hf, qi, false, tt);
                float mt = tt[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mt = fmaxf(mt, tt[r]);
                const float mn = fmaxf(m_run, mt);
                if (mn != -INFINITY) {
                    float sum = 0.0f;
#pragma unroll
                    for (int r = 0; r < 16; ++r) sum += fast_exp2(tt[r] - mn);
                    l_run = l_run * fast_exp2(m_run - mn) + sum;
                    m_run = mn;
                }
            }
        }
        store_k(buf ^ 1);
        mcur = mpre;
        __syncthreads();
        const int t2 = min(t + 2, ntiles - 1);
        load_k(t2);
        mpre.load(a, mr, mrow_off, t2 * BN, hf);
    }
    {  // the two half-waves holding the same query row
        const float m_o = __shfl_xor(m_run, 32);
        const float l_o = __shfl_xor(l_run, 32);
        const float mn = fmaxf(m_run, m_o);
        if (mn != -INFINITY) {
            l_run = l_run * fast_exp2(m_run - mn) + l_o * fast_exp2(m_o - mn);
            m_run = mn;
        }
    }
    const bool dead = (m_run == -INFINITY);
    const float lse2 = dead ? INFINITY : m_run + __log2f(l_run);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dead ? -INFINITY : lse2 * LN2), lr,
                                          pred(row_ok && hf == 0, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.l_s[2] * 4)),
                                          0, 0);

    // ---------------- sweep 2: P = exp2(t - lse2), store, O^T += V^T P^T
    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};

    __syncthreads();  // sweep 1 readers are done with both LDS buffers
    if (ntiles > 0) {
        load_k(0);
        load_v(0);
        mpre.load(a, mr, mrow_off, 0, hf);
        store_k(0);
        store_vt(0);
        mcur = mpre;
        __syncthreads();
        const int t1 = min(1, ntiles - 1);
        load_k(t1);
        load_v(t1);
        mpre.load(a, mr, mrow_off, t1 * BN, hf);
    }
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * BN;
        const int buf = t & 1;
        if (a.causal && k0 > qw + 31) {
            // whole tile above this wave's diagonal: P is zero, O unchanged
            const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < 4; ++c) store8<T, VEC>(pr, prow_off, row_ok, k0 + 16 * c + 8 * hf, a.Skv, z);
        } else {
            const bool edge = (k0 + BN > a.Skv) || (a.causal && k0 + BN - 1 > qw);
            f32x16 acc2[2];
            qk_tile(buf, acc2);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float mv[16];
                mcur.get(a, mr, mrow_off, k0, hf, kb, mv);
                float tt[16];
                if (edge) scores16<MASK>(a, acc2[kb], mv, k0 + 32 * kb, hf, qi, true, tt);
                else scores16<MASK>(a, acc2[kb], mv, k0 + 32 * kb, hf, qi, false, tt);
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = fast_exp2(tt[r] - lse2);
                store8<T, VEC>(pr, prow_off, row_ok, k0 + 32 * kb + 8 * hf, a.Skv, p);
                store8<T, VEC>(pr, prow_off, row_ok, k0 + 32 * kb + 16 + 8 * hf, a.Skv, p + 8);
                if constexpr (SZ == 2) {
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        const vec pv = TR::cvt8(p + 8 * c2);
#pragma unroll
                        for (int d = 0; d < ND; ++d) {
                            const vec va = as_vec<T>(*reinterpret_cast<const u32x4*>(
                                &vt_lds[buf][(32 * d + swap23(n)) * VLD + 32 * kb + 16 * c2 + 8 * hf]));
                            oacc[d] = TR::mfma(va, pv, oacc[d]);
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
#pragma unroll
                        for (int d = 0; d < ND; ++d) {
                            const float va = vt_lds[buf][(32 * d + swap23(n)) * VLD + 32 * kb + kk(hf, r)];
                            oacc[d] = TR::mfma(va, p[r], oacc[d]);
                        }
                    }
                }
            }
        }
        store_k(buf ^ 1);
        store_vt(buf ^ 1);
        mcur = mpre;
        __syncthreads();
        const int t2 = min(t + 2, ntiles - 1);
        load_k(t2);
        load_v(t2);
        mpre.load(a, mr, mrow_off, t2 * BN, hf);
    }

    // ---------------- O: lane (n, h) holds O[qi][32d + 8h ..+8) and [32d + 16 + 8h ..+8)
    {
        const uint32_t orow_off = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.o_s[2] * SZ);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = oacc[d][r];
            store8<T, VEC>(orr, orow_off, row_ok, 32 * d + 8 * hf, D, x);
            store8<T, VEC>(orr, orow_off, row_ok, 32 * d + 16 + 8 * hf, D, x + 8);
        }
    }

    // ---------------- causal: keys past this workgroup's last row are zero
    zero_rows<T, VEC>(pr, a.p_s[2], qw, a.Sq, ntiles * BN, a.Skv, lane);
}

template <typename T, int D, int NW, bool VEC>
static int launch_twopass_mask(int mask_kind, const FwdArgs& a, hipStream_t s) {
    dim3 grid(a.n_blocks), block(NW * 64);
    switch (mask_kind) {
        case MASK_NONE: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_NONE, VEC>), grid, block, 0, s, a); break;
        case MASK_BOOL: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_BOOL, VEC>), grid, block, 0, s, a); break;
        case MASK_ADD: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_ADD, VEC>), grid, block, 0, s, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// Element-wise layouts only need correctness: they get one two-wave shape.
template <typename T>
static int launch_twopass_t(int D, int mask_kind, int waves, bool vec, const FwdArgs& a, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define SDPA_TP_DIM(DD)                                                                   \
    case DD:                                                                              \
        if (!vec) return launch_twopass_mask<T, DD, 2, false>(mask_kind, a, s);           \
        if (waves == 4) return launch_twopass_mask<T, DD, 4, true>(mask_kind, a, s);      \
        if (waves == 2) return launch_twopass_mask<T, DD, 2, true>(mask_kind, a, s);      \
        return (int)hipErrorInvalidValue;
    switch (D) {
        SDPA_TP_DIM(32)
        SDPA_TP_DIM(64)
        SDPA_TP_DIM(128)
        default: return (int)hipErrorInvalidValue;
    }
#undef SDPA_TP_DIM
}

}  // namespace sdpa
