// Fused single-sweep kernel for shapes with few score tiles.
//
// FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton + P800
// exact-P/A1)", single-kernel fusion and threshold sections: when a row block
// has few score tiles, one launch that keeps the block's scores on chip
// computes Q K^T once (the two-sweep kernel computes it twice) and reads the
// mask once. The math is the same as the two-sweep kernel's: exact row
// maximum and sum, LSE, P = exp(scale*QK^T - LSE) rounded to the dtype, and
// O accumulated from the rounded P ("P800 exact-P fast path" update).
//
// Workgroup = 32 query rows of one (batch, head) and NW waves (1..8); wave w
// owns keys [w*kpw, (w+1)*kpw) and holds their scores (S^T blocks of 32 keys,
// the same MFMA layout as the two-sweep kernel) in registers. Row maximum and
// sum are combined across waves through LDS. Each wave then stages its own V
// rows in LDS by buffer-to-LDS loads and accumulates a partial O^T; the
// partials are summed through LDS. Every global load (Q, K, mask, V) is
// issued before the first store, so no wait ever covers a store.

#include <mutex>
#include <set>
#include <utility>

#include "sdpa_device.h"

namespace sdpa {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x2 lds_tr16(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

// vmcnt(0) only
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// lgkmcnt(0) only
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Largest number of 32-key score blocks one wave keeps in registers.
template <int D>
constexpr int fused_max_blocks() {
    return D == 128 ? FUSED_MAX_KEYS_PER_WAVE_D128 / 32 : FUSED_MAX_KEYS_PER_WAVE / 32;
}

// Bytes of dynamic LDS for `nw` waves: per wave a 32-row V block or, later, a
// 32 x (D + 4) float partial O^T; then the row max and sum of every wave.
template <typename T, int D>
constexpr int fused_lds_bytes(int nw) {
    return nw * 32 * (D + 4) * 4 + 2 * nw * 32 * 4;
}

template <typename T, int D, int MASK, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 512)))
void sdpa_fused_kernel(const FwdArgs a) {
    using TR = Tr<T>;
    using vec = typename TR::vec;
    constexpr int SZ = (int)sizeof(T);
    constexpr int KH = TR::KH;
    constexpr int KSTEP = 2 * KH;
    constexpr int NKS = D / KSTEP;
    constexpr int ND = D / 32;
    constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;
    constexpr int ROWB = D * SZ;
    constexpr int CPR = ROWB / 16;
    constexpr int NBMAX = fused_max_blocks<D>();
    constexpr int OPITCH = D + 4;  // floats per partial-O row (padding spreads the banks)
    static_assert(CPR % 4 == 0, "V block layout needs a multiple of 4 chunks per row");

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nw = (int)(blockDim.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31;
    const int hf = lane >> 5;
    float* red_m = reinterpret_cast<float*>(smem + nw * 32 * OPITCH * 4);
    float* red_l = red_m + nw * 32;
    uint8_t* vblk = smem + wave * 32 * ROWB;

    const Work w = decode_block(blockIdx.x, a);
    const int hk = w.hq / a.group;
    const int q0 = w.qblk * 32;
    const int qi = q0 + n;
    const bool row_ok = qi < a.Sq;
    // keys any row of this block may keep
    const int kend = a.causal ? min(a.Skv, max(0, q0 + 32 + a.coff)) : a.Skv;
    const int kpw = a.keys_per_wave;
    const int kbase = wave * kpw;
    const int nb = max(0, min((kend - kbase + 31) / 32, kpw / 32));

    const rsrc_t qr = make_rsrc(static_cast<const T*>(a.q) + w.b * a.q_s[0] + w.hq * a.q_s[1], a.q_ext);
    const rsrc_t kr = make_rsrc(static_cast<const T*>(a.k) + w.b * a.k_s[0] + hk * a.k_s[1], a.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(a.v) + w.b * a.v_s[0] + hk * a.v_s[1], a.v_ext);
    const rsrc_t pr = make_rsrc(static_cast<T*>(a.p) + w.b * a.p_s[0] + w.hq * a.p_s[1], a.p_ext);
    const rsrc_t orr = make_rsrc(static_cast<T*>(a.o) + w.b * a.o_s[0] + w.hq * a.o_s[1], a.o_ext);
    const rsrc_t lr = make_rsrc(a.lse + w.b * a.l_s[0] + w.hq * a.l_s[1], a.l_ext);
    rsrc_t mr = kr;
    if constexpr (MASK != MASK_NONE)
        mr = make_rsrc(static_cast<const uint8_t*>(a.mask) + (w.b * a.m_s[0] + w.hq * a.m_s[1]) * ME, a.m_ext);
    const uint32_t krow_bytes = (uint32_t)(a.k_s[2] * SZ);
    const uint32_t vrow_bytes = (uint32_t)(a.v_s[2] * SZ);
    const uint32_t prow = pred(row_ok, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.p_s[2] * SZ));

    // Q fragments (B operand): lane (n, h) holds Q[qi][c*KSTEP + h*KH .. +KH)
    vec qf[NKS];
    {
        const uint32_t qoff = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.q_s[2] * SZ);
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            const uint32_t off = pred(row_ok, qoff + (uint32_t)((c * KSTEP + hf * KH) * SZ));
            if constexpr (sizeof(T) == 2) qf[c] = as_vec<T>(ld128(qr, off));
            else qf[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, off, 0, 0));
        }
    }

    // ---------------- scores of this wave's keys (base 2, masked), kept in registers
    const int kr0 = swap23(n);
    f32x16 s[NBMAX];
    float m_loc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NBMAX; ++kb) {
        s[kb] = f32x16{};
        if (kb < nb) {
            const int jb = kbase + 32 * kb;
            // A operand: K row jb + swap23(m), elements c*KSTEP + h*KH .. +KH (rows past Skv read 0)
            const int krow = jb + kr0;
            const uint32_t kro = pred(krow < a.Skv, (uint32_t)krow * krow_bytes);
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < NKS; ++c) {
                const uint32_t off = kro == OOB ? OOB : kro + (uint32_t)((c * KSTEP + hf * KH) * SZ);
                vec ka;
                if constexpr (sizeof(T) == 2) ka = as_vec<T>(ld128(kr, off));
                else ka = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kr, off, 0, 0));
                acc = TR::mfma(ka, qf[c], acc);
            }
            float mv[16];
            if constexpr (MASK != MASK_NONE)
                load_mask16<T, MASK, VEC>(a, mr, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.m_s[2] * ME), jb, hf, mv);
            const bool edge = (jb + 32 > a.Skv) || (a.causal && jb + 31 > q0 + a.coff);
            float t[16];
            scores16<MASK>(a, acc, mv, jb, hf, qi, edge, t);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = t[r];
                m_loc = fmaxf(m_loc, t[r]);
            }
        }
    }

    // ---------------- row maximum and sum across the waves
    m_loc = fmaxf(m_loc, __shfl_xor(m_loc, 32));
    if (hf == 0) red_m[wave * 32 + n] = m_loc;
    __syncthreads();
    float M = -INFINITY;
    for (int i = 0; i < nw; ++i) M = fmaxf(M, red_m[i * 32 + n]);
    float l_loc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int kb = 0; kb < NBMAX; ++kb)
            if (kb < nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) l_loc += fast_exp2(s[kb][r] - M);
            }
    }
    l_loc += __shfl_xor(l_loc, 32);
    if (hf == 0) red_l[wave * 32 + n] = l_loc;
    __syncthreads();
    float L = 0.0f;
    for (int i = 0; i < nw; ++i) L += red_l[i * 32 + n];
    const bool dead = (M == -INFINITY);
    // dead rows: lse2 = +inf makes every probability exp2(-inf) = +0
    const float lse2 = dead ? INFINITY : M + __log2f(L);

    // ---------------- probabilities (rounded to the dtype) and O^T += V^T P^T
    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
    vec pv[NBMAX][2];  // 16-bit: the rounded probabilities of each block, two runs of 8

    // transposing-read address of the V^T operand (as in the two-sweep kernel)
    const int trg = lane >> 4, trs = lane & 15;
    const int tr_sig = ((trs & 1) << 1) | ((trs >> 1) & 1);
    const int tr_row = 8 * (trg >> 1) + (trs >> 2);
    const int tr_col = 16 * (trg & 1) + 4 * tr_sig;
    // V block layout: 16-row x 4-chunk bricks of 16-byte chunks
    auto pos_v = [](int row, int chunk) -> int {
        return (row >> 4) * (16 * CPR) + (chunk >> 2) * 64 + 4 * (row & 15) + (chunk & 3);
    };

#pragma unroll
    for (int kb = 0; kb < NBMAX; ++kb) {
        if (kb < nb) {
            const int jb = kbase + 32 * kb;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(s[kb][r] - lse2);
            if constexpr (sizeof(T) == 2) {
                pv[kb][0] = TR::cvt8(p);
                pv[kb][1] = TR::cvt8(p + 8);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = p[r];
            }
            // stage V rows jb .. jb+31 of this wave (the previous block's reads are done)
            wait_lds();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int j = 0; j < CPR / 2; ++j) {
                const int row = 16 * (j / (CPR / 4)) + (lane >> 2);
                const int chunk = 4 * (j % (CPR / 4)) + (lane & 3);
                const uint32_t vo = pred(jb + row < a.Skv, (uint32_t)(jb + row) * vrow_bytes + (uint32_t)(chunk * 16));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vblk + j * 1024), 16, vo, 0, 0, 0);
            }
            wait_vmem();
            asm volatile("" ::: "memory");
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    // the rounded probabilities plus their rounded residual:
                    // O accumulates P to twice the dtype's precision
                    const vec pl = TR::lo8(p + 8 * c2, pv[kb][c2]);
                    vec va[ND];
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        u32x2 h2[2];
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            const int row = 16 * c2 + tr_row + 4 * r;
                            const int col = 32 * d + tr_col;
                            h2[r] = lds_tr16(vblk + pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
                        }
                        va[d] = __builtin_bit_cast(vec, u32x4{h2[0][0], h2[0][1], h2[1][0], h2[1][1]});
                    }
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[d], pv[kb][c2], oacc[d]);
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[d], pl, oacc[d]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = kk(hf, r);
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const int col = 32 * d + swap23(n);
                        const float va = *reinterpret_cast<const float*>(
                            vblk + pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
                        oacc[d] = TR::mfma(va, s[kb][r], oacc[d]);
                    }
                }
            }
        }
    }

    // ---------------- stores: P of this wave's keys, zeros past them, LSE
#pragma unroll
    for (int kb = 0; kb < NBMAX; ++kb) {
        if (kb < nb) {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int j = kbase + 32 * kb + 16 * c2 + 8 * hf;
                if constexpr (sizeof(T) == 2) {
                    const u32x4 bits = __builtin_bit_cast(u32x4, pv[kb][c2]);
                    if constexpr (VEC) {
                        st128(pr, pred(j < a.Skv, prow + (uint32_t)(j * SZ)), bits);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(bits[e >> 1] >> (16 * (e & 1))), pr,
                                                                  pred(row_ok && j + e < a.Skv, prow + (uint32_t)((j + e) * SZ)),
                                                                  0, 0);
                    }
                } else {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = s[kb][8 * c2 + e];
                    store8<T, VEC>(pr, row_ok ? prow : 0u, row_ok, j, a.Skv, x);
                }
            }
        }
    }
    {
        const int c0 = min(a.Skv, kbase + 32 * nb);
        const int c1 = wave == nw - 1 ? a.Skv : min(a.Skv, kbase + kpw);
        zero_rows<T, VEC>(pr, a.p_s[2], q0, a.Sq, c0, c1, lane);
    }
    if (wave == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dead ? -INFINITY : lse2 * LN2), lr,
                                              pred(row_ok && hf == 0, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.l_s[2] * 4)),
                                              0, 0);

    // ---------------- O: lane (n, h) holds O^T columns 32d + kk(h, r) of row n
    if (nw == 1) {
        const uint32_t orow = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.o_s[2] * SZ);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = oacc[d][r];
            store8<T, VEC>(orr, orow, row_ok, 32 * d + 8 * hf, D, x);
            store8<T, VEC>(orr, orow, row_ok, 32 * d + 16 + 8 * hf, D, x + 8);
        }
        return;
    }
    __syncthreads();  // every wave is done with its V block
    float* opart = reinterpret_cast<float*>(smem) + wave * 32 * OPITCH;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) opart[n * OPITCH + 32 * d + kk(hf, r)] = oacc[d][r];
    __syncthreads();
    const float* obase = reinterpret_cast<const float*>(smem);
    for (int i = threadIdx.x; i < 32 * (D / 8); i += nw * 64) {
        const int row = i / (D / 8), c8 = i - row * (D / 8);
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        for (int ww = 0; ww < nw; ++ww) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] += obase[(ww * 32 + row) * OPITCH + 8 * c8 + e];
        }
        const int orow_i = q0 + row;
        const bool ok = orow_i < a.Sq;
        store8<T, VEC>(orr, (uint32_t)((int64_t)(ok ? orow_i : 0) * a.o_s[2] * SZ), ok, 8 * c8, D, x);
    }
}

// ---------------------------------------------------------------- wide variant
//
// Workgroup = RG row groups of 32 query rows (a.fused_rg) x KG key groups;
// wave w = (row group w / KG, key group w % KG) scores 32 rows against
// a.keys_per_wave keys, held in registers as above. The V rows of the
// workgroup's whole key range are staged in LDS by whole-row buffer-to-LDS
// loads and shared by the row groups (the two-level split lets a short-query
// shape fill the chip with half as many workgroups); V rows then replace
// them, landing while the row statistics are combined. Whole-row loads cost
// the memory pipeline about a quarter of what the MFMA-layout accesses (32
// rows x 32 bytes per instruction) cost. Row maximum and sum are combined
// over the KG waves of a row group through LDS; once V has landed no load is
// left in flight, so each block's probabilities are stored as soon as they
// are made.

// Bytes of dynamic LDS of the wide kernel: the staged V rows (or, after
// them, the partial O^T of every wave; with `oseq`, one O^T accumulation
// buffer per row group; none with one key group per row group, whose waves
// store their outputs directly), then the row max and sum of every wave.
template <typename T, int D>
constexpr int fused_wide_lds_bytes(int nw, int rg, int vrows, bool oseq) {
    const int v = vrows * D * (int)sizeof(T), o = nw == rg ? 0 : (oseq ? rg : nw) * 32 * (D + 4) * 4;
    return (v > o ? v : o) + 2 * nw * 32 * 4;
}

template <typename T, int D>
constexpr int fused_wide_max_blocks() {
    return fused_wide_max_keys(sizeof(T) == 4 ? DT_F32 : DT_F16, D) / 32;
}

// RANGE: the workgroup takes one key range of a long-key call (range r of
// a.n_splits: keys [r * R, r * R + R), R = KG * a.keys_per_wave) as a call of
// its own, and writes, instead of P, O and LSE: its probabilities relative
// to its own row maximum (float32, ws_e), its rows' (max, sum) (ws_ml) and
// its float32 partial O (ws_o); sdpa_range_combine_kernel folds them.
template <typename T, int D, int MASK, bool VEC, bool RANGE>
__global__ __launch_bounds__(FUSED_MAX_WAVES * 64) void sdpa_fused_wide_kernel(const FwdArgs a_in) {
    static_assert(!RANGE || VEC, "key ranges take the 16-byte layouts");
    using TR = Tr<T>;
    using vec = typename TR::vec;
    constexpr int SZ = (int)sizeof(T);
    constexpr int KH = TR::KH;
    constexpr int KSTEP = 2 * KH;
    constexpr int NKS = D / KSTEP;
    constexpr int ND = D / 32;
    constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;
    constexpr int ROWB = D * SZ;
    constexpr int CPR = ROWB / 16;
    constexpr int NBMAX = fused_wide_max_blocks<T, D>();
    constexpr int OPITCH = D + 4;
    static_assert(CPR % 4 == 0, "V block layout needs a multiple of 4 chunks per row");

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    FwdArgs ra = a_in;  // RANGE: rebased onto the workgroup's key range below
    const FwdArgs& a = RANGE ? ra : a_in;
    const int nw = (int)(blockDim.x >> 6);
    const int RG = a.fused_rg;
    const int KG = nw / RG;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31;
    const int hf = lane >> 5;
    const int rg = wave / KG, kg = wave - (wave / KG) * KG;
    const int kpw = a.keys_per_wave;
    const int vrows = KG * kpw;  // staged V rows: keys 0 .. vrows-1 (zeros past Skv)
    const int obytes = KG == 1 ? 0 : (a.fused_oseq ? RG : nw) * 32 * OPITCH * 4;
    const int vbytes = vrows * ROWB > obytes ? vrows * ROWB : obytes;
    float* red_m = reinterpret_cast<float*>(smem + vbytes);
    float* red_l = red_m + nw * 32;

    // workgroup -> (batch, head, row block); each XCD (ids handed out in
    // turn) takes a contiguous range, so the row blocks of a head, and the
    // heads of a KV group, read K and V through one L2
    int L = blockIdx.x;
    if ((a.n_blocks & 7) == 0) {
        const int per = a.n_blocks >> 3;
        L = (L & 7) * per + (L >> 3);
    }
    int range = 0, koff = 0;
    if constexpr (RANGE) {
        if (a_in.fused_hg) {
            // the group's heads are this workgroup's row groups
            range = L % a_in.n_splits;
            L /= a_in.n_splits;
        } else {
            // workgroup order: the query heads of a KV group fastest, then the
            // ranges, so that a group's heads read each range's K and V rows
            // through L2 at about the same time; L becomes (batch, head, row block)
            const int g = L % a_in.group;
            L /= a_in.group;
            range = L % a_in.n_splits;
            L /= a_in.n_splits;
            const int rb0 = L % a_in.n_qblk, bk = L / a_in.n_qblk;  // bk = batch * Hkv + KV head
            L = ((bk / a_in.Hkv) * a_in.Hq + (bk % a_in.Hkv) * a_in.group + g) * a_in.n_qblk + rb0;
        }
        // the range's keys as a call of its own: K, V and mask columns from
        // koff on (the descriptors shrink by as much), Skv the range's keys,
        // the causal offset moved with them
        koff = range * vrows;
        ra.Skv = min(vrows, a_in.Skv - koff);
        ra.coff = a_in.coff - koff;
        const int64_t kadv = (int64_t)koff * a_in.k_s[2], vadv = (int64_t)koff * a_in.v_s[2];
        ra.k = static_cast<const T*>(a_in.k) + kadv;
        ra.v = static_cast<const T*>(a_in.v) + vadv;
        ra.k_ext = a_in.k_ext - (uint32_t)(kadv * SZ);
        ra.v_ext = a_in.v_ext - (uint32_t)(vadv * SZ);
        if constexpr (MASK != MASK_NONE) {
            const int64_t madv = (int64_t)koff * a_in.m_s[3] * ME;
            ra.mask = static_cast<const uint8_t*>(a_in.mask) + madv;
            ra.m_ext = a_in.m_ext - (uint32_t)madv;
        }
    }
    // (batch, query head of this wave, row block). Head row groups
    // (a.fused_hg): the RG row groups are RG query heads of one KV group, all
    // on the same 32 rows, so the group's K and V rows are staged once; else
    // they are consecutive 32-row groups of one head.
    const bool hgr = a.fused_hg != 0;
    const int rb = L % a.n_qblk;
    int b, hq;
    if (hgr) {
        const int nset = a.group / RG;  // head sets per KV group
        const int hs = L / a.n_qblk;    // (batch * Hkv + KV head) * nset + set
        const int bk = hs / nset;
        b = bk / a.Hkv;
        hq = (bk - b * a.Hkv) * a.group + (hs - bk * nset) * RG + rg;
    } else {
        const int bh = L / a.n_qblk;
        b = bh / a.Hq;
        hq = bh - b * a.Hq;
    }
    const int hk = hq / a.group;
    const int q0 = hgr ? rb * 32 : (rb * RG + rg) * 32;
    const int qi = q0 + n;
    const bool row_ok = qi < a.Sq;
    // keys the rows of this row group (and of the whole workgroup) may keep
    const int kend = a.causal ? min(a.Skv, max(0, q0 + 32 + a.coff)) : a.Skv;
    const int kend_wg = a.causal ? min(a.Skv, max(0, (hgr ? rb + 1 : (rb + 1) * RG) * 32 + a.coff)) : a.Skv;
    const int kbase = kg * kpw;
    const int nb = max(0, min((kend - kbase + 31) / 32, kpw / 32));

    const rsrc_t qr = make_rsrc(static_cast<const T*>(a.q) + b * a.q_s[0] + hq * a.q_s[1], a.q_ext);
    const rsrc_t kr = make_rsrc(static_cast<const T*>(a.k) + b * a.k_s[0] + hk * a.k_s[1], a.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(a.v) + b * a.v_s[0] + hk * a.v_s[1], a.v_ext);
    // RANGE: float32 probability rows of this (batch, head) in ws_e (pitch
    // Skv of the whole call, from the range's first key), partial O rows in
    // ws_o (pitch D)
    const int64_t wsrow0 = (int64_t)(b * a.Hq + hq) * a.Sq;  // first workspace row of this (batch, head)
    const rsrc_t pr = RANGE ? make_rsrc(a_in.ws_e + wsrow0 * a_in.Skv + koff,
                                        (uint32_t)(((int64_t)a.Sq * a_in.Skv - koff) * 4))
                            : make_rsrc(static_cast<T*>(a.p) + b * a.p_s[0] + hq * a.p_s[1], a.p_ext);
    // output rows of query head h of this workgroup's batch
    auto o_rsrc = [&](int h) -> rsrc_t {
        if constexpr (RANGE)
            return make_rsrc(a_in.ws_o + ((int64_t)range * a.B * a.Hq * a.Sq + (int64_t)(b * a.Hq + h) * a.Sq) * D,
                             (uint32_t)((int64_t)a.Sq * D * 4));
        else
            return make_rsrc(static_cast<T*>(a.o) + b * a.o_s[0] + h * a.o_s[1], a.o_ext);
    };
    const rsrc_t orr = o_rsrc(hq);
    const rsrc_t lr = make_rsrc(a.lse + b * a.l_s[0] + hq * a.l_s[1], a.l_ext);
    rsrc_t mr = kr;
    if constexpr (MASK != MASK_NONE)
        mr = make_rsrc(static_cast<const uint8_t*>(a.mask) + (b * a.m_s[0] + hq * a.m_s[1]) * ME, a.m_ext);
    const uint32_t krow_bytes = (uint32_t)(a.k_s[2] * SZ);
    const uint32_t vrow_bytes = (uint32_t)(a.v_s[2] * SZ);
    const uint32_t prow = RANGE ? pred(row_ok, (uint32_t)((int64_t)(row_ok ? qi : 0) * a_in.Skv * 4))
                                : pred(row_ok, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.p_s[2] * SZ));
    // one run of 8 output columns of a row: the dtype, or float32 partials (RANGE)
    auto store_o8 = [&](rsrc_t r, uint32_t row_off, bool ok, int col, const float* x) __attribute__((always_inline)) {
        if constexpr (RANGE) store8<float, true>(r, row_off, ok, col, D, x);
        else store8<T, VEC>(r, row_off, ok, col, D, x);
    };
    const int64_t o_pitch = RANGE ? D : a.o_s[2];  // output row pitch, elements
    constexpr int OSZ = RANGE ? 4 : SZ;

    // ---------------- K rows of the workgroup's keys into LDS (V replaces them
    // once the scores are made): buffer-to-LDS loads of whole rows.
    // K layout: row-major, chunk c of row r at r * CPR + (c ^ fk(r)), so that
    // the operand reads (16 consecutive rows, one chunk each) are free of
    // bank conflicts; instruction i fills chunk positions [64 i, 64 i + 64).
    // V layout: 16-row x 4-chunk bricks, read by the transposing LDS read.
    constexpr int RPI = 64 / CPR;  // rows per buffer-to-LDS instruction
    constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;
    auto fk = [](int row) -> int { return (row / RPB) & (CPR - 1); };
    auto pos_k = [&](int row, int chunk) -> int { return row * CPR + (chunk ^ fk(row)); };
    auto pos_v = [](int row, int chunk) -> int {
        return (row >> 4) * (16 * CPR) + (chunk >> 2) * 64 + 4 * (row & 15) + (chunk & 3);
    };
    const int nstage = (min(kend_wg, vrows) + 31) / 32 * 32;  // staged rows (whole 32-key blocks)
    {
        const int nki = nstage / RPI;
        for (int i = wave; i < nki; i += nw) {
            const int row = i * RPI + lane / CPR;
            const int chunk = (lane % CPR) ^ fk(row);
            const uint32_t ko = pred(row < a.Skv, (uint32_t)row * krow_bytes + (uint32_t)(chunk * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(smem + i * 1024), 16, ko, 0, 0, 0);
        }
    }

    // Q fragments (B operand): lane (n, h) holds Q[qi][c*KSTEP + h*KH .. +KH)
    vec qf[NKS];
    {
        const uint32_t qoff = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.q_s[2] * SZ);
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            const uint32_t off = pred(row_ok, qoff + (uint32_t)((c * KSTEP + hf * KH) * SZ));
            if constexpr (sizeof(T) == 2) qf[c] = as_vec<T>(ld128(qr, off));
            else qf[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, off, 0, 0));
        }
    }

    // ---------------- scores of this wave's keys (base 2, masked), kept in
    // registers; K operands from LDS. The raw mask words of each 32-key block
    // are loaded two blocks ahead into a ring of three register sets (loads
    // past the wave's last block are aimed outside the buffers and return
    // zeros).
    const int kr0 = swap23(n);
    constexpr int MQ = !VEC || MASK == MASK_NONE ? 0 : MASK == MASK_BOOL ? 1 : SZ == 2 ? 2 : 4;
    constexpr int RING = MQ > 0 ? 3 : 1;
    u32x4 mring[RING][MQ > 0 ? MQ : 1];
    const uint32_t mrow = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.m_s[2] * ME);
    auto issue_mask = [&](int kb, int slot) __attribute__((always_inline)) {
        if constexpr (MQ > 0) {
            const bool live = kb < nb;
            const int jb = kbase + 32 * kb;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = jb + 16 * c + 8 * hf;
                const uint32_t off = pred(live && j < a.Skv, mrow + (uint32_t)j * ME);
                if constexpr (MASK == MASK_BOOL) {
                    const u32x2 w = ld64(mr, off);
                    mring[slot][0][2 * c] = w[0];
                    mring[slot][0][2 * c + 1] = w[1];
                } else if constexpr (SZ == 2) {
                    mring[slot][c] = ld128(mr, off);
                } else {
                    mring[slot][2 * c] = ld128(mr, off);
                    mring[slot][2 * c + 1] = ld128(mr, off == OOB ? OOB : off + 16);
                }
            }
        }
    };
    // base-2 mask terms of a block from its raw words (the vector layouts of load_mask16)
    auto mask_terms = [&](int slot, float* mv) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if constexpr (MASK == MASK_BOOL) {
                const uint32_t w0 = mring[slot][0][2 * c], w1 = mring[slot][0][2 * c + 1];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    mv[8 * c + e] = (((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xffu) ? 0.0f : -INFINITY;
            } else if constexpr (SZ == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = mring[slot][c][e >> 1];
                    mv[8 * c + e] = Tr<T>::to_f((w >> (16 * (e & 1))) & 0xffffu) * LOG2E;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t b0 = mring[slot][2 * c][e], b1 = mring[slot][2 * c + 1][e];
                    mv[8 * c + e] = __builtin_bit_cast(float, b0) * LOG2E;
                    mv[8 * c + 4 + e] = __builtin_bit_cast(float, b1) * LOG2E;
                }
            }
        }
    };
    if constexpr (RING > 1) {
#pragma unroll
        for (int kb = 0; kb < RING - 1 && kb < NBMAX; ++kb) issue_mask(kb, kb);
    }
    // every wave's K rows have landed (this wave's by the wait, the others' by
    // the barrier after theirs)
    wait_vmem();
    __syncthreads();
    f32x16 s[NBMAX];
    float m_loc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NBMAX; ++kb) {
        if constexpr (RING > 1) {
            if (kb + RING - 1 < NBMAX) issue_mask(kb + RING - 1, (kb + RING - 1) % RING);
        }
        s[kb] = f32x16{};
        if (kb < nb) {
            const int jb = kbase + 32 * kb;
            // K operand (A), k-step c: lane (m, h) reads row jb + swap23(m),
            // elements c*KSTEP + h*KH .. +KH; all reads of the block before its chain
            vec ka[NKS];
#pragma unroll
            for (int c = 0; c < NKS; ++c) {
                const int elem = c * KSTEP + hf * KH;
                const uint8_t* kp = smem + pos_k(jb + kr0, elem * SZ / 16) * 16 + ((elem * SZ) & 15);
                if constexpr (sizeof(T) == 2) ka[c] = as_vec<T>(*reinterpret_cast<const u32x4*>(kp));
                else ka[c] = *reinterpret_cast<const float*>(kp);
            }
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < NKS; ++c) acc = TR::mfma(ka[c], qf[c], acc);
            float mv[16];
            if constexpr (MQ > 0) mask_terms(kb % RING, mv);
            else if constexpr (MASK != MASK_NONE) load_mask16<T, MASK, VEC>(a, mr, mrow, jb, hf, mv);
            const bool edge = (jb + 32 > a.Skv) || (a.causal && jb + 31 > q0 + a.coff);
            float t[16];
            scores16<MASK>(a, acc, mv, jb, hf, qi, edge, t);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = t[r];
                m_loc = fmaxf(m_loc, t[r]);
            }
        }
    }

    // ---------------- row maximum and sum across the key groups of the row group
    m_loc = fmaxf(m_loc, __shfl_xor(m_loc, 32));
    if (hf == 0) red_m[wave * 32 + n] = m_loc;
    __syncthreads();  // (every wave is also done reading the staged K rows)
    // ---------------- V rows into the same LDS region, landing while the row
    // statistics are combined
    {
        const int nvi = nstage / 32 * (CPR / 2);
        for (int i = wave; i < nvi; i += nw) {
            const int vb = i / (CPR / 2), j = i - (i / (CPR / 2)) * (CPR / 2);
            const int row = 32 * vb + 16 * (j / (CPR / 4)) + (lane >> 2);
            const int chunk = 4 * (j % (CPR / 4)) + (lane & 3);
            const uint32_t vo = pred(row < a.Skv, (uint32_t)row * vrow_bytes + (uint32_t)(chunk * 16));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(smem + vb * 32 * ROWB + j * 1024), 16, vo, 0, 0, 0);
        }
    }
    float M = -INFINITY;
    for (int i = 0; i < KG; ++i) M = fmaxf(M, red_m[(rg * KG + i) * 32 + n]);
    float l_loc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int kb = 0; kb < NBMAX; ++kb)
            if (kb < nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) l_loc += fast_exp2(s[kb][r] - M);
            }
    }
    l_loc += __shfl_xor(l_loc, 32);
    if (hf == 0) red_l[wave * 32 + n] = l_loc;
    // every wave's V loads have landed (this wave's by the wait; the others'
    // by the barrier after theirs)
    wait_vmem();
    __syncthreads();
    float Lsum = 0.0f;
    for (int i = 0; i < KG; ++i) Lsum += red_l[(rg * KG + i) * 32 + n];
    const bool dead = (M == -INFINITY);
    // RANGE: probabilities relative to the range's row maximum (the combine
    // launch scales them by 2^(M - lse2) once every range's sum is known)
    const float lse2 = dead ? INFINITY : RANGE ? M : M + __log2f(Lsum);

    // ---------------- probabilities (rounded to the dtype), stored as made, and O^T += V^T P^T
    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
    const int trg = lane >> 4, trs = lane & 15;
    const int tr_sig = ((trs & 1) << 1) | ((trs >> 1) & 1);
    const int tr_row = 8 * (trg >> 1) + (trs >> 2);
    const int tr_col = 16 * (trg & 1) + 4 * tr_sig;
#pragma unroll
    for (int kb = 0; kb < NBMAX; ++kb) {
        if (kb < nb) {
            const int jb = kbase + 32 * kb;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(s[kb][r] - lse2);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const vec pv = TR::cvt8(p + 8 * c2);
                    const int j = jb + 16 * c2 + 8 * hf;
                    const u32x4 bits = __builtin_bit_cast(u32x4, pv);
                    if constexpr (RANGE) {
                        store8<float, true>(pr, row_ok ? prow : 0u, row_ok, j, a.Skv, p + 8 * c2);
                    } else if constexpr (VEC) {
                        st128(pr, pred(j < a.Skv, prow + (uint32_t)(j * SZ)), bits);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(bits[e >> 1] >> (16 * (e & 1))), pr,
                                                                  pred(row_ok && j + e < a.Skv, prow + (uint32_t)((j + e) * SZ)),
                                                                  0, 0);
                    }
                    // the rounded probabilities plus their rounded residual:
                    // O accumulates P to twice the dtype's precision
                    const vec pl = TR::lo8(p + 8 * c2, pv);
                    vec va[ND];
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        u32x2 h2[2];
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            const int row = jb + 16 * c2 + tr_row + 4 * r;
                            const int col = 32 * d + tr_col;
                            h2[r] = lds_tr16(smem + pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
                        }
                        va[d] = __builtin_bit_cast(vec, u32x4{h2[0][0], h2[0][1], h2[1][0], h2[1][1]});
                    }
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[d], pv, oacc[d]);
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[d], pl, oacc[d]);
                }
            } else {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
                    store8<T, VEC>(pr, row_ok ? prow : 0u, row_ok, jb + 16 * c2 + 8 * hf, a.Skv, p + 8 * c2);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = jb + kk(hf, r);
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const int col = 32 * d + swap23(n);
                        const float va = *reinterpret_cast<const float*>(
                            smem + pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
                        oacc[d] = TR::mfma(va, p[r], oacc[d]);
                    }
                }
            }
        }
    }

    // ---------------- zeros past this wave's keys, LSE
    {
        const int c0 = min(a.Skv, kbase + 32 * nb);
        const int c1 = kg == KG - 1 ? a.Skv : min(a.Skv, kbase + kpw);
        if constexpr (RANGE) zero_rows<float, true>(pr, a_in.Skv, q0, a.Sq, c0, c1, lane);
        else zero_rows<T, VEC>(pr, a.p_s[2], q0, a.Sq, c0, c1, lane);
    }
    if constexpr (RANGE) {
        if (kg == 0 && hf == 0 && row_ok)
            a_in.ws_ml[(int64_t)range * a.B * a.Hq * a.Sq + wsrow0 + qi] = float2{M, dead ? 0.0f : Lsum};
    } else if (kg == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dead ? -INFINITY : lse2 * LN2), lr,
                                              pred(row_ok && hf == 0, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.l_s[2] * 4)),
                                              0, 0);
    }

    // ---------------- O: the KG partial O^T of each row group summed through LDS
    if (KG == 1) {
        const uint32_t orow = (uint32_t)((int64_t)(row_ok ? qi : 0) * o_pitch * OSZ);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = oacc[d][r];
            store_o8(orr, orow, row_ok, 32 * d + 8 * hf, x);
            store_o8(orr, orow, row_ok, 32 * d + 16 + 8 * hf, x + 8);
        }
        return;
    }
    __syncthreads();  // every wave is done reading the staged V rows
    // The KG partial O^T of each row group summed in key-group order: every
    // wave's partial in LDS, then summed by the reading threads; or, with
    // a.fused_oseq (less LDS: one buffer per row group), accumulated in turn
    // (key group 0 writes, the others add) -- the same sums either way.
    const bool oseq = a.fused_oseq != 0;
    if (oseq) {
        float* obuf = reinterpret_cast<float*>(smem) + rg * 32 * OPITCH;
        for (int k2 = 0; k2 < KG; ++k2) {
            if (kg == k2) {
#pragma unroll
                for (int d = 0; d < ND; ++d)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float* o = obuf + n * OPITCH + 32 * d + kk(hf, r);
                        *o = (k2 == 0 ? 0.0f : *o) + oacc[d][r];
                    }
            }
            __syncthreads();
        }
    } else {
        float* opart = reinterpret_cast<float*>(smem) + wave * 32 * OPITCH;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) opart[n * OPITCH + 32 * d + kk(hf, r)] = oacc[d][r];
        __syncthreads();
    }
    const float* obase = reinterpret_cast<const float*>(smem);
    for (int i = threadIdx.x; i < RG * 32 * (D / 8); i += nw * 64) {
        const int rr = i / (D / 8), c8 = i - (i / (D / 8)) * (D / 8);
        const int g = rr >> 5, row = rr & 31;
        float x[8];
        if (oseq) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = obase[(g * 32 + row) * OPITCH + 8 * c8 + e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            for (int ww = 0; ww < KG; ++ww) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] += obase[((g * KG + ww) * 32 + row) * OPITCH + 8 * c8 + e];
            }
        }
        const int orow_i = hgr ? rb * 32 + row : (rb * RG + g) * 32 + row;
        const bool ok = orow_i < a.Sq;
        store_o8(hgr ? o_rsrc(hq - rg + g) : orr, (uint32_t)((int64_t)(ok ? orow_i : 0) * o_pitch * OSZ), ok, 8 * c8, x);
    }
}

// Output of a call whose keys ran as ranges of the wide kernel: per row, the
// log-sum-exp from every range's (max, sum); P = RNE(e * c_r) with e the
// range's float32 probability and c_r = 2^(max_r - lse2); O the sum over
// ranges of c_r times the range's float32 partial O, rounded once.
// Workgroup = one row x 2048 keys (8 per thread). The row's statistics are
// reduced over the workgroup's threads (a fixed tree: the same bits in every
// workgroup of the row) and the scales c_r kept in LDS; each workgroup also
// sums the partial outputs of a slice of the head dim (threads split over
// ranges, then a fixed-order sum through LDS), so that no thread walks every
// range. Keys past the last range (causal) get P = 0.
template <bool MAX>
__device__ __forceinline__ float block_reduce256(float x, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = MAX ? fmaxf(x, y) : x + y;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    x = MAX ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return x;
}

template <typename T>
__global__ __launch_bounds__(256) void sdpa_range_combine_kernel(const FwdArgs a, int D, int range_keys, int nchunk) {
    constexpr int SZ = (int)sizeof(T);
    __shared__ float cs[RANGE_MAX];
    __shared__ float red[256];
    const int tid = (int)threadIdx.x;
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    const int64_t row = (int64_t)blockIdx.x / nchunk;
    const int chunk = (int)((int64_t)blockIdx.x - row * nchunk);
    const int n = a.n_splits;
    const float2* st = a.ws_ml + row;  // range r's (max, sum) at st[r * rows]
    float m = -INFINITY;
    for (int r = tid; r < n; r += 256) m = fmaxf(m, st[(int64_t)r * rows].x);
    const float M = block_reduce256<true>(m, red);
    const bool dead = (M == -INFINITY);
    float l = 0.0f;
    if (!dead)
        for (int r = tid; r < n; r += 256) {
            const float2 s = st[(int64_t)r * rows];
            if (s.x != -INFINITY) l += s.y * fast_exp2(s.x - M);
        }
    const float lsum = block_reduce256<false>(l, red);
    const float lse2 = dead ? INFINITY : M + __log2f(lsum);
    // scale of range r's probabilities and partial output (0 for a range
    // that keeps no key of the row, and for a dead row)
    for (int r = tid; r < n; r += 256) {
        const float mr = st[(int64_t)r * rows].x;
        cs[r] = mr == -INFINITY ? 0.0f : fast_exp2(mr - lse2);
    }
    __syncthreads();
    const int q = (int)(row % a.Sq);
    const int64_t bh = row / a.Sq;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const int j0 = (chunk * 256 + tid) * 8;
    if (j0 < a.Skv) {
        const int r = j0 / range_keys;  // a run of 8 keys lies in one range (multiples of 32)
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (r < n) {
            const float c = cs[r];
            const float* e = a.ws_e + row * a.Skv + j0;
            const f32x4 u0 = *reinterpret_cast<const f32x4*>(e);
            const f32x4 u1 = *reinterpret_cast<const f32x4*>(e + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = u0[i] * c;
                x[4 + i] = u1[i] * c;
            }
        }
        T* p = static_cast<T*>(a.p) + b * a.p_s[0] + h * a.p_s[1] + (int64_t)q * a.p_s[2] + j0;
        if constexpr (SZ == 2) {
            *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, Tr<T>::cvt8(x));
        } else {
            *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
        }
    }
    // O columns [d0, d0 + dn) of this workgroup: thread (g, col) sums ranges
    // g, g + G, ... of column d0 + col; then the G partial sums in order
    const int dpc = (D + nchunk - 1) / nchunk;  // columns per workgroup (<= D <= 256)
    const int d0 = chunk * dpc;
    const int dn = min(D, d0 + dpc) - d0;
    T* orow = static_cast<T*>(a.o) + b * a.o_s[0] + h * a.o_s[1] + (int64_t)q * a.o_s[2];
    if (dn > 0) {
        const int G = 256 / dpc;
        const int col = tid % dpc, g = tid / dpc;
        float x = 0.0f;
        if (col < dn && g < G)
            for (int r = g; r < n; r += G) x += cs[r] * a.ws_o[((int64_t)r * rows + row) * D + d0 + col];
        red[tid] = x;
        __syncthreads();
        if (tid < dn) {
            float s = 0.0f;
            for (int gg = 0; gg < G; ++gg) s += red[gg * dpc + tid];
            if constexpr (SZ == 2) {
                orow[d0 + tid] = static_cast<T>(s);
            } else {
                orow[d0 + tid] = s;
            }
        }
    }
    if (chunk == 0 && tid == 0) a.lse[b * a.l_s[0] + h * a.l_s[1] + (int64_t)q * a.l_s[2]] = dead ? -INFINITY : lse2 * LN2;
}

// Allow a kernel the most dynamic LDS any fused launch asks for, once per
// (device, kernel): a host-side function attribute, so later launches (also
// those recorded into a graph) make no further runtime call for it.
int raise_lds_limit(const void* k) {
    static std::mutex mu;
    static std::set<std::pair<int, const void*>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({dev, k})) return 0;
    e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, FUSED_LDS_MAX);
    if (e == hipSuccess) done.insert({dev, k});
    return (int)e;
}

template <typename T, int D, bool VEC>
int launch_fused_t(int mask_kind, int waves, const FwdArgs& a, hipStream_t s) {
    const dim3 grid(a.n_blocks), block(waves * 64);
    const bool wide = a.fused_rg > 0;
    const bool ranges = wide && a.n_splits > 1;  // key ranges of the wide kernel, then the combine
    if (ranges && !VEC) return (int)hipErrorInvalidValue;
    const size_t lds = wide ? (size_t)fused_wide_lds_bytes<T, D>(waves, a.fused_rg, waves / a.fused_rg * a.keys_per_wave,
                                                                  a.fused_oseq != 0)
                            : (size_t)fused_lds_bytes<T, D>(waves);
#define SDPA_FUSED_LAUNCH(MK)                                                                               \
    {                                                                                                       \
        auto* k = ranges ? sdpa_fused_wide_kernel<T, D, MK, VEC, VEC>                                      \
                  : wide ? sdpa_fused_wide_kernel<T, D, MK, VEC, false> : sdpa_fused_kernel<T, D, MK, VEC>;  \
        if (lds > 64 * 1024) {                                                                              \
            const int e = raise_lds_limit(reinterpret_cast<const void*>(k));                                 \
            if (e != 0) return e;                                                                           \
        }                                                                                                   \
        hipLaunchKernelGGL(k, grid, block, lds, s, a);                                                      \
        break;                                                                                              \
    }
    switch (mask_kind) {
        case MASK_NONE: SDPA_FUSED_LAUNCH(MASK_NONE)
        case MASK_BOOL: SDPA_FUSED_LAUNCH(MASK_BOOL)
        case MASK_ADD: SDPA_FUSED_LAUNCH(MASK_ADD)
        default: return (int)hipErrorInvalidValue;
    }
#undef SDPA_FUSED_LAUNCH
    if (ranges) {
        const int range_keys = waves / a.fused_rg * a.keys_per_wave;
        const int nchunk = (a.Skv + 2047) / 2048;
        const int64_t nwg = (int64_t)a.B * a.Hq * a.Sq * nchunk;
        hipLaunchKernelGGL(sdpa_range_combine_kernel<T>, dim3((unsigned)nwg), dim3(256), 0, s, a, D, range_keys, nchunk);
    }
    return (int)hipGetLastError();
}

template <typename T>
int launch_fused_dt(int D, int mask_kind, int waves, bool vec, const FwdArgs& a, hipStream_t s) {
    switch (D) {
        case 32: return vec ? launch_fused_t<T, 32, true>(mask_kind, waves, a, s) : launch_fused_t<T, 32, false>(mask_kind, waves, a, s);
        case 64: return vec ? launch_fused_t<T, 64, true>(mask_kind, waves, a, s) : launch_fused_t<T, 64, false>(mask_kind, waves, a, s);
        case 128: return vec ? launch_fused_t<T, 128, true>(mask_kind, waves, a, s) : launch_fused_t<T, 128, false>(mask_kind, waves, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_fused(int dtype, int D, int mask_kind, int waves, bool vec, const FwdArgs& a, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (waves < 1 || waves > FUSED_MAX_WAVES || a.keys_per_wave % 32 != 0 || a.keys_per_wave <= 0)
        return (int)hipErrorInvalidValue;
    if (a.fused_rg > 0) {
        // wide variant: RG row groups x KG key groups, every staged V row in LDS
        if (waves % a.fused_rg != 0 || a.keys_per_wave > fused_wide_max_keys(dtype, D) ||
            fused_wide_lds_bytes_rt(dtype, D, waves, a.fused_rg, waves / a.fused_rg * a.keys_per_wave, a.fused_oseq != 0) >
                FUSED_LDS_MAX ||
            (a.fused_hg && (a.group % a.fused_rg != 0)))
            return (int)hipErrorInvalidValue;
    } else {
        const int maxk = D == 128 ? FUSED_MAX_KEYS_PER_WAVE_D128 : FUSED_MAX_KEYS_PER_WAVE;
        if (a.keys_per_wave > maxk) return (int)hipErrorInvalidValue;
    }
    if (a.n_splits > 1) {
        // key ranges: the wide kernel on 16-byte layouts, its workspace given,
        // every range starting inside the keys, whole ranges per row block
        const int64_t rk = a.fused_rg > 0 ? (int64_t)(waves / a.fused_rg) * a.keys_per_wave : 0;
        if (a.fused_rg <= 0 || !vec || !a.ws_ml || !a.ws_o || !a.ws_e || (int64_t)(a.n_splits - 1) * rk >= a.Skv ||
            a.n_blocks % a.n_splits != 0 || a.Skv % 8 != 0 || a.n_splits > RANGE_MAX)
            return (int)hipErrorInvalidValue;
    }
    switch (dtype) {
        case DT_F32: return launch_fused_dt<float>(D, mask_kind, waves, vec, a, s);
        case DT_F16: return launch_fused_dt<_Float16>(D, mask_kind, waves, vec, a, s);
        case DT_BF16: return launch_fused_dt<__bf16>(D, mask_kind, waves, vec, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace sdpa
