// gfx950 kernels for the materialised-probability SDPA forward.
//
// Math (FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton +
// P800 exact-P/A1)", "P800 exact-P fast path" update): with the row-wise
// log-sum-exp known, P = exp(scale * Q K^T - LSE) is exact, so a first sweep
// over the keys finds LSE and a second sweep writes P and accumulates
// O = P V. Scores live in the base-2 domain (scale * log2 e folded into one
// multiplier, as the cudnn-frontend merge-log notes do for their kernels).
//
// Layout trick used everywhere: each wave computes S^T = K Q^T for 32 keys x
// 32 queries with v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2_f32 for
// float32). Lane l owns query column n = l % 32 and half h = l / 32. Loading
// MFMA row m of the K operand from key swap23(m) (bits 2 and 3 exchanged)
// makes accumulator register r of lane (n, h) hold key
//     kk(h, r) = r < 8 ? 8h + r : 16 + 8h + (r - 8)
// so each lane ends up with two runs of 8 consecutive keys of ONE query row:
//   * the row statistics are lane-local plus one exchange with lane l ^ 32;
//   * the rounded P values are already the B operand of the next MFMA,
//     O^T += V^T P^T (keys 16c + 8h .. +7 in slot order), with no LDS round
//     trip;
//   * every lane stores P as 16-byte row chunks.
// V^T is staged in LDS (keys contiguous per head-dim row) so that the A
// operand of O^T += V^T P^T is one 16-byte LDS read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_internal.h"

namespace sdpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BN = TILE_N;  // keys per tile (two 32-key MFMA blocks)

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ constexpr int kk(int h, int r) { return r < 8 ? 8 * h + r : 16 + 8 * h + (r - 8); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- element traits

template <typename T> struct Tr;

template <> struct Tr<__bf16> {
    static constexpr int KH = 8;  // operand elements per lane per MFMA
    using vec = bf16x8;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec cvt8(const float* x) {
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(f, vec);
    }
    static __device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
};

template <> struct Tr<_Float16> {
    static constexpr int KH = 8;
    using vec = f16x8;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec cvt8(const float* x) {
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(f, vec);
    }
    static __device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }
};

template <> struct Tr<float> {
    static constexpr int KH = 1;
    using vec = float;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f(float x) { return x; }
};

template <typename T>
__device__ __forceinline__ typename Tr<T>::vec load_op(const T* p) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(typename Tr<T>::vec, *reinterpret_cast<const u32x4*>(p));
    } else {
        return *p;
    }
}

template <typename T>
__device__ __forceinline__ typename Tr<T>::vec zero_op() {
    if constexpr (sizeof(T) == 2) {
        return __builtin_bit_cast(typename Tr<T>::vec, u32x4{0u, 0u, 0u, 0u});
    } else {
        return 0.0f;
    }
}

// ---------------------------------------------------------------- block mapping

struct Work {
    int b, hq, qblk;
};

// Workgroup ids go round-robin over the 8 XCDs, each with its own L2. Remap so
// that one XCD receives a contiguous range of logical ids: all query blocks of
// a (batch, head), and the heads sharing a KV head, then hit the same L2 for
// K and V. Causal calls list the heaviest (last) query blocks first.
__device__ __forceinline__ Work decode_block(int L, const FwdArgs& a) {
    const int nb = a.n_blocks;
    const int nfull = nb & ~7;
    int logical = L;
    if (L < nfull) logical = (L & 7) * (nfull >> 3) + (L >> 3);
    const int bh = logical / a.n_qblk;
    const int r = logical - bh * a.n_qblk;
    Work w;
    w.qblk = a.causal ? (a.n_qblk - 1 - r) : r;
    w.b = bh / a.Hq;
    w.hq = bh - w.b * a.Hq;
    return w;
}

// ---------------------------------------------------------------- masks

// Mask values for the 16 keys lane (n, h) holds in one 32-key block, as
// floats in the base-2 domain (additive) or 0/1 keep flags (bool).
template <typename T, int MASK>
__device__ __forceinline__ void load_mask16(const FwdArgs& a, const void* mrow, int j0, float* out) {
    // keys j0 + [0..8) and j0 + 16 + [0..8)
    if constexpr (MASK == MASK_BOOL) {
        const uint8_t* m = reinterpret_cast<const uint8_t*>(mrow);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int j = j0 + 16 * c;
            if (a.mask_vec && j + 8 <= a.Skv) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(m + j);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[8 * c + e] = ((w[e >> 2] >> (8 * (e & 3))) & 0xffu) ? 1.0f : 0.0f;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    out[8 * c + e] = (j + e < a.Skv && m[(int64_t)(j + e) * a.m_s[3]]) ? 1.0f : 0.0f;
            }
        }
    } else if constexpr (MASK == MASK_ADD) {
        const T* m = reinterpret_cast<const T*>(mrow);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int j = j0 + 16 * c;
            if constexpr (sizeof(T) == 2) {
                if (a.mask_vec && j + 8 <= a.Skv) {
                    const typename Tr<T>::vec w = load_op<T>(m + j);
#pragma unroll
                    for (int e = 0; e < 8; ++e) out[8 * c + e] = (float)w[e] * LOG2E;
                    continue;
                }
            } else {
                if (a.mask_vec && j + 8 <= a.Skv) {
                    const f32x4 w0 = *reinterpret_cast<const f32x4*>(m + j);
                    const f32x4 w1 = *reinterpret_cast<const f32x4*>(m + j + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        out[8 * c + e] = w0[e] * LOG2E;
                        out[8 * c + 4 + e] = w1[e] * LOG2E;
                    }
                    continue;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                out[8 * c + e] = (j + e < a.Skv) ? Tr<T>::to_f(m[(int64_t)(j + e) * a.m_s[3]]) * LOG2E : 0.0f;
        }
    }
}

// Scaled, masked scores of one S^T block in the base-2 domain; -inf where a
// key is removed (causal, mask, or past the end of the keys).
template <typename T, int MASK>
__device__ __forceinline__ void scores16(const FwdArgs& a, const f32x16& acc, int jblk, int hf, int qi,
                                         bool edge, const void* mrow, float* t) {
    float mv[16];
    if constexpr (MASK != MASK_NONE) load_mask16<T, MASK>(a, mrow, jblk + 8 * hf, mv);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float x = acc[r] * a.scale_log2;
        if constexpr (MASK == MASK_ADD) x = x + mv[r];
        bool drop = false;
        if constexpr (MASK == MASK_BOOL) drop = mv[r] == 0.0f;
        if (edge) {
            const int j = jblk + kk(hf, r);
            drop = drop || j >= a.Skv || (a.causal && j > qi);
        }
        t[r] = drop ? -INFINITY : x;
    }
}

// ---------------------------------------------------------------- stores

template <typename T>
__device__ __forceinline__ void store8(T* row, int j, int limit, bool vec_ok, const float* x) {
    // x[0..8) -> row[j .. j+8), clipped at `limit`
    if constexpr (sizeof(T) == 2) {
        const typename Tr<T>::vec v = Tr<T>::cvt8(x);
        if (vec_ok && j + 8 <= limit) {
            *reinterpret_cast<u32x4*>(row + j) = __builtin_bit_cast(u32x4, v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (j + e < limit) row[j + e] = v[e];
        }
    } else {
        if (vec_ok && j + 8 <= limit) {
            *reinterpret_cast<f32x4*>(row + j) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4*>(row + j + 4) = f32x4{x[4], x[5], x[6], x[7]};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (j + e < limit) row[j + e] = x[e];
        }
    }
}

// Zero P[row][c0 .. c1) with the 64 lanes of a wave writing 16-byte chunks.
template <typename T>
__device__ __forceinline__ void zero_cols(T* row, int c0, int c1, bool vec_ok, int lane) {
    constexpr int E = 16 / sizeof(T);
    if (vec_ok) {
        for (int j = c0 + lane * E; j < c1; j += 64 * E) {
            if (j + E <= c1) {
                *reinterpret_cast<u32x4*>(row + j) = u32x4{0u, 0u, 0u, 0u};
            } else {
                for (int e = 0; j + e < c1; ++e) row[j + e] = T(0);
            }
        }
    } else {
        for (int j = c0 + lane; j < c1; j += 64) row[j] = T(0);
    }
}

// ---------------------------------------------------------------- two-pass kernel

// One workgroup: NW waves x 32 query rows of one (batch, query head). K (and
// V^T in the second sweep) tiles of 64 keys are staged through LDS once and
// shared by all waves; the next tile is prefetched into registers while the
// current one is consumed.
template <typename T, int D, int NW, int MASK>
__global__ __launch_bounds__(NW * 64) void sdpa_twopass_kernel(const FwdArgs a) {
    using TR = Tr<T>;
    using vec = typename TR::vec;
    constexpr int KH = TR::KH;
    constexpr int KSTEP = 2 * KH;
    constexpr int NKS = D / KSTEP;          // MFMAs per 32x32 score block
    constexpr int NT = NW * 64;
    constexpr int QB = 32 * NW;
    constexpr int E16 = 16 / sizeof(T);     // elements per 16-byte chunk
    constexpr int KLD = D + E16;            // LDS row pitch of the K tile
    constexpr int VLD = BN + E16;           // LDS row pitch of the V^T tile
    constexpr int CPR = D / E16;            // 16-byte chunks per K/V row
    constexpr int KCH = (BN * CPR + NT - 1) / NT;        // K chunks per thread
    constexpr int VIT = ((BN / 4) * CPR + NT - 1) / NT;  // V items (4 keys x 1 chunk) per thread
    constexpr int ND = D / 32;              // 32-wide head-dim chunks of O^T

    __shared__ __attribute__((aligned(16))) T k_lds[BN * KLD];
    __shared__ __attribute__((aligned(16))) T vt_lds[D * VLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    const T* qbase = reinterpret_cast<const T*>(a.q) + w.b * a.q_s[0] + w.hq * a.q_s[1];
    const T* kbase = reinterpret_cast<const T*>(a.k) + w.b * a.k_s[0] + hk * a.k_s[1];
    const T* vbase = reinterpret_cast<const T*>(a.v) + w.b * a.v_s[0] + hk * a.v_s[1];
    T* prow = reinterpret_cast<T*>(a.p) + w.b * a.p_s[0] + w.hq * a.p_s[1] + (int64_t)qi * a.p_s[2];
    const void* mrow = nullptr;
    if constexpr (MASK != MASK_NONE) {
        const int64_t off = w.b * a.m_s[0] + w.hq * a.m_s[1] + (int64_t)(row_ok ? qi : 0) * a.m_s[2];
        if constexpr (MASK == MASK_BOOL) mrow = reinterpret_cast<const uint8_t*>(a.mask) + off;
        else mrow = reinterpret_cast<const T*>(a.mask) + off;
    }

    // Q fragments (B operand): lane (n, h) holds Q[qi][c*KSTEP + h*KH .. +KH)
    vec qf[NKS];
#pragma unroll
    for (int c = 0; c < NKS; ++c)
        qf[c] = row_ok ? load_op<T>(qbase + (int64_t)qi * a.q_s[2] + c * KSTEP + hf * KH) : zero_op<T>();

    // Causal: keys past this workgroup's last row are zero for all its rows.
    // Issue those stores first so they drain while the first sweep computes.
    if (ntiles * BN < a.Skv) {
        T* wrow0 = reinterpret_cast<T*>(a.p) + w.b * a.p_s[0] + w.hq * a.p_s[1];
        for (int r = 0; r < 32; ++r) {
            const int row = qw + r;
            if (row >= a.Sq) break;
            zero_cols<T>(wrow0 + (int64_t)row * a.p_s[2], ntiles * BN, a.Skv, a.p_vec, lane);
        }
    }

    u32x4 kreg[KCH];
    u32x4 vreg[VIT][4];

    auto load_k = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            kreg[i] = u32x4{0u, 0u, 0u, 0u};
            if (c < BN * CPR) {
                const int row = c / CPR, ch = c - row * CPR;
                if (k0 + row < a.Skv)
                    kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(k0 + row) * a.k_s[2] + ch * E16);
            }
        }
    };
    auto store_k = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            if (c < BN * CPR) {
                const int row = c / CPR, ch = c - row * CPR;
                *reinterpret_cast<u32x4*>(&k_lds[row * KLD + ch * E16]) = kreg[i];
            }
        }
    };
    auto load_v = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
            const int it = tid + i * NT;
#pragma unroll
            for (int r = 0; r < 4; ++r) vreg[i][r] = u32x4{0u, 0u, 0u, 0u};
            if (it < (BN / 4) * CPR) {
                const int kg = it / CPR, ch = it - kg * CPR;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 4 * kg + r;
                    if (key < a.Skv)
                        vreg[i][r] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * a.v_s[2] + ch * E16);
                }
            }
        }
    };
    auto store_vt = [&]() {
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
            const int it = tid + i * NT;
            if (it < (BN / 4) * CPR) {
                const int kg = it / CPR, ch = it - kg * CPR;
                if constexpr (sizeof(T) == 2) {
                    // 8 head-dim rows, each receiving 4 consecutive keys (8 bytes)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int wd = e >> 1;
                        uint32_t x0 = vreg[i][0][wd], x1 = vreg[i][1][wd], x2 = vreg[i][2][wd], x3 = vreg[i][3][wd];
                        uint32_t lo, hi;
                        if (e & 1) {
                            lo = (x0 >> 16) | (x1 & 0xffff0000u);
                            hi = (x2 >> 16) | (x3 & 0xffff0000u);
                        } else {
                            lo = (x0 & 0xffffu) | (x1 << 16);
                            hi = (x2 & 0xffffu) | (x3 << 16);
                        }
                        *reinterpret_cast<u32x2*>(&vt_lds[(ch * 8 + e) * VLD + 4 * kg]) = u32x2{lo, hi};
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<u32x4*>(&vt_lds[(ch * 4 + e) * VLD + 4 * kg]) =
                            u32x4{vreg[i][0][e], vreg[i][1][e], vreg[i][2][e], vreg[i][3][e]};
                }
            }
        }
    };

    // S^T block kb (keys 32kb .. 32kb+31 of the staged tile) for this wave's queries.
    auto qk_block = [&](int kb) {
        f32x16 acc = {};
        const T* kr = &k_lds[(32 * kb + swap23(n)) * KLD + hf * KH];
#pragma unroll
        for (int c = 0; c < NKS; ++c) acc = TR::mfma(load_op<T>(kr + c * KSTEP), qf[c], acc);
        return acc;
    };

    // ---------------- sweep 1: row maximum and sum (base 2)
    float m_run = -INFINITY, l_run = 0.0f;
    if (ntiles > 0) load_k(0);
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * BN;
        __syncthreads();
        store_k();
        __syncthreads();
        if (t + 1 < ntiles) load_k(t + 1);
        const bool edge = (k0 + BN > a.Skv) || (a.causal && k0 + BN - 1 > qw);
        if (a.causal && k0 > qw + 31) continue;  // whole tile above this wave's diagonal
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x16 acc = qk_block(kb);
            float tt[16];
            scores16<T, MASK>(a, acc, k0 + 32 * kb, hf, qi, edge, mrow, tt);
            float mt = tt[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = fmaxf(mt, tt[r]);
            const float mn = fmaxf(m_run, mt);
            if (mn != -INFINITY) {
                float s = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) s += fast_exp2(tt[r] - mn);
                l_run = l_run * fast_exp2(m_run - mn) + s;
                m_run = mn;
            }
        }
    }
    // combine the two half-waves that share a query row
    {
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
    if (row_ok && hf == 0)
        a.lse[w.b * a.l_s[0] + w.hq * a.l_s[1] + (int64_t)qi * a.l_s[2]] = dead ? -INFINITY : lse2 * LN2;

    // ---------------- sweep 2: P = exp2(t - lse2), store, O^T += V^T P^T
    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};

    if (ntiles > 0) {
        load_k(0);
        load_v(0);
    }
    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * BN;
        __syncthreads();
        store_k();
        store_vt();
        __syncthreads();
        if (t + 1 < ntiles) {
            load_k(t + 1);
            load_v(t + 1);
        }
        const bool edge = (k0 + BN > a.Skv) || (a.causal && k0 + BN - 1 > qw);
        if (a.causal && k0 > qw + 31) {
            // whole tile above this wave's diagonal: P is zero, O unchanged
            if (row_ok) {
                const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c) store8<T>(prow, k0 + 16 * c + 8 * hf, a.Skv, a.p_vec, z);
            }
            continue;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x16 acc = qk_block(kb);
            float tt[16];
            scores16<T, MASK>(a, acc, k0 + 32 * kb, hf, qi, edge, mrow, tt);
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(tt[r] - lse2);
            if (row_ok) {
                store8<T>(prow, k0 + 32 * kb + 8 * hf, a.Skv, a.p_vec, p);
                store8<T>(prow, k0 + 32 * kb + 16 + 8 * hf, a.Skv, a.p_vec, p + 8);
            }
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const vec pv = TR::cvt8(p + 8 * c2);
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const vec va = load_op<T>(&vt_lds[(32 * d + swap23(n)) * VLD + 32 * kb + 16 * c2 + 8 * hf]);
                        oacc[d] = TR::mfma(va, pv, oacc[d]);
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const float va = vt_lds[(32 * d + swap23(n)) * VLD + 32 * kb + kk(hf, r)];
                        oacc[d] = TR::mfma(va, p[r], oacc[d]);
                    }
                }
            }
        }
    }

    // ---------------- O store: lane (n, h) holds O[qi][32d + 8h ..+8) and [32d + 16 + 8h ..+8)
    if (row_ok) {
        T* orow = reinterpret_cast<T*>(a.o) + w.b * a.o_s[0] + w.hq * a.o_s[1] + (int64_t)qi * a.o_s[2];
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = oacc[d][r];
            store8<T>(orow, 32 * d + 8 * hf, D, a.o_vec, x);
            store8<T>(orow, 32 * d + 16 + 8 * hf, D, a.o_vec, x + 8);
        }
    }
}

// ---------------------------------------------------------------- launchers

template <typename T, int D, int NW>
static int launch_tp_mask(int mask_kind, const FwdArgs& a, hipStream_t s) {
    dim3 grid(a.n_blocks), block(NW * 64);
    switch (mask_kind) {
        case MASK_NONE: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_NONE>), grid, block, 0, s, a); break;
        case MASK_BOOL: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_BOOL>), grid, block, 0, s, a); break;
        case MASK_ADD: hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MASK_ADD>), grid, block, 0, s, a); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

template <typename T, int D>
static int launch_tp_waves(int waves, int mask_kind, const FwdArgs& a, hipStream_t s) {
    switch (waves) {
        case 2: return launch_tp_mask<T, D, 2>(mask_kind, a, s);
        case 4: return launch_tp_mask<T, D, 4>(mask_kind, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

template <typename T>
static int launch_tp_dim(int D, int waves, int mask_kind, const FwdArgs& a, hipStream_t s) {
    switch (D) {
        case 32: return launch_tp_waves<T, 32>(waves, mask_kind, a, s);
        case 64: return launch_tp_waves<T, 64>(waves, mask_kind, a, s);
        case 128: return launch_tp_waves<T, 128>(waves, mask_kind, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

int launch_twopass(int dtype, int D, int mask_kind, int waves, const FwdArgs& a, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case DT_F32: return launch_tp_dim<float>(D, waves, mask_kind, a, s);
        case DT_F16: return launch_tp_dim<_Float16>(D, waves, mask_kind, a, s);
        case DT_BF16: return launch_tp_dim<__bf16>(D, waves, mask_kind, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

int launch_fused(int, int, int, int, const FwdArgs&, void*) { return (int)hipErrorNotSupported; }

}  // namespace sdpa
