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
// Workgroup = NW compute waves (32 query rows each, one (batch, query head))
// plus one loader wave (or four compute waves that share the loads, NL). The
// loader wave copies each tile of K (64 keys; 32 with a bool mask), and of V
// and the mask in sweep 2, from global memory straight into LDS with
// buffer-to-LDS loads, double-buffered, one barrier per tile. The compute
// waves issue no global loads inside the loops, so their probability stores
// are never waited for: on this hardware a wait for a load also waits for
// every store issued before it, and the probability map is most of the
// traffic. The LDS tile layouts make every operand read a per-lane base plus
// a constant offset, free of bank conflicts; the V^T operand of
// O^T += V^T P^T is read with the gfx950 transposing LDS read
// (ds_read_b64_tr_b16). For few query rows against many keys the same kernel
// runs over key ranges (SPL), with a combine kernel for O.

#pragma once

#include <type_traits>

#include "sdpa_device.h"

// lambdas of the kernels below are always inlined: one that became a call
// would put the arrays it captures by reference (accumulators) in scratch
#define SDPA_INLINE __attribute__((always_inline))

namespace sdpa {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read: within each 16-lane group, output lane 4a+b receives
// element b of the 4-element reads made by source lanes 4j+a, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

// vmcnt(0) only (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// NL: no loader wave; the compute waves share the tile loads (and defer
// each tile's probability stores by one tile, see the kernel).
// CT (bool masks without a loader wave): mask tiles are staged in sweep 1
// only, in the V buffers that sweep leaves free; sweep 2 takes each tile's
// class from a per-wave record and reads the mask from memory for mixed
// tiles only. No LDS of its own for the mask. HR (head rows): the waves
// share 32 query rows, so a mask tile has 32 rows.
template <typename T, int D, int NW, int MASK, bool VEC, int TN, bool NL, bool CT = false, bool HR = false>
struct TwoPassCfg {
    static constexpr int NWAVES = NL ? NW : NW + 1;  // waves per workgroup
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int BN = TN;                 // keys per tile: 32 or 64 (one or two MFMA blocks)
    static constexpr int NKB = TN / 32;
    static constexpr int QB = 32 * NW;            // query rows per workgroup
    static constexpr int ROWB = D * SZ;           // bytes per K/V row
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per K/V row
    static constexpr int RPI = 64 / CPR;          // tile rows per buffer-to-LDS instruction
    static constexpr int NI = BN / RPI;           // instructions per K (or V) tile
    static constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;  // rows per 64-bank span
    static constexpr int TILEB = BN * ROWB;       // bytes per K (or V) tile
    static constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;
    static constexpr bool MLDS = MASK != MASK_NONE && VEC;  // mask tiles staged in LDS
    static constexpr int MROWB = BN * ME;         // bytes per mask tile row
    static constexpr int MCPR = MROWB / 16;
    static constexpr int MRPI = 64 / MCPR;
    static constexpr int MQ = HR ? 32 : QB;       // mask tile rows
    static constexpr int MNI = MQ / MRPI;
    static constexpr int MTILEB = MLDS ? MQ * MROWB : 0;
    static constexpr bool CT_FITS = MTILEB <= TILEB;  // a mask tile fits in a V buffer
    // Probabilities of a tile are staged per wave in LDS and written out as
    // whole rows (the MFMA layout gives each lane two 16-byte runs of one
    // row per 32 keys, i.e. 32-byte pieces of 32 rows per store: the costly
    // pattern for the memory pipeline). Staged only while two workgroups
    // still fit in one CU's LDS.
    static constexpr int ZC = BN * SZ / 16;       // 16-byte chunks per row of a P tile
    static constexpr int ZRPB = ZC * 16 >= 256 ? 1 : 256 / (ZC * 16);  // P rows per 64-bank span
    static constexpr int PSTB = 32 * BN * SZ;     // bytes of one wave's staged P tile
    static constexpr int KVM_BYTES = 2 * (2 * TILEB + (CT ? 0 : MTILEB));
    static constexpr bool PSTAGE = VEC && KVM_BYTES + NW * PSTB <= 80 * 1024;
    static constexpr int LDS_BYTES = KVM_BYTES + (PSTAGE ? NW * PSTB : 0);

    // LDS tile layouts, in 16-byte chunk positions: row-major, with the
    // chunks of each row permuted by an XOR (chunk c of row r at position
    // r * CPR + (c ^ f(r))). Each buffer-to-LDS instruction then fetches whole
    // rows (a few cache lines, the cheap pattern for the memory pipeline),
    // and the operand reads are free of bank conflicts:
    //  K: 16 consecutive rows, one chunk each (ds_read_b128): f spreads the
    //     rows sharing a 256-byte bank window over distinct chunk slots;
    //  V: 4 rows x 2 chunks per 16-lane group of the transposing read, the
    //     two groups of a cycle on the other 2 chunks: f moves whole groups
    //     of 4 chunks.
    static __device__ __forceinline__ int fk(int row) { return (row / RPB) & (CPR - 1); }
    static __device__ __forceinline__ int fv(int row) { return 4 * ((row / RPB) & (CPR / 4 - 1)); }
    static __device__ __forceinline__ int pos_k(int row, int chunk) { return row * CPR + (chunk ^ fk(row)); }
    static __device__ __forceinline__ int pos_v(int row, int chunk) { return row * CPR + (chunk ^ fv(row)); }
    // staged P tile: row-major, chunks XOR-permuted like K (writes: 16 rows,
    // one chunk each; reads: whole rows)
    static __device__ __forceinline__ int pos_p(int row, int chunk) {
        return row * ZC + (chunk ^ ((row / ZRPB) & (ZC - 1)));
    }
    static_assert(CPR % 4 == 0, "tile layouts need a multiple of 4 chunks per row");
};

#ifndef SDPA_TP_WPE
#define SDPA_TP_WPE(NW) ((NW) >= 4 ? 3 : 2)
#endif

// SPL: 0 the whole call; with key ranges (loader-wave kernels only) 1 runs
// sweep 1 over this workgroup's range and writes its rows' (max, sum), 2
// folds every range's statistics into the LSE, runs sweep 2 over its range
// (final P) and writes a float32 partial O.
// Packed variable-length sequences: rebase a copy of the arguments onto
// sequence b. The host leaves the batch strides 0 and Sq / Skv at the
// maximum lengths; the sequence's token range comes from cu_seqlens, clamped
// to the packed tensors (and its lengths to the maxima), so no access leaves
// them whatever the offsets hold.
template <typename T>
__device__ __forceinline__ void thd_rebase(FwdArgs& a, int b) {
    const int q0 = min(max(a.cu_q[b], 0), a.Tq);
    const int q1 = min(max(a.cu_q[b + 1], q0), a.Tq);
    const int k0 = min(max(a.cu_k[b], 0), a.Tkv);
    const int k1 = min(max(a.cu_k[b + 1], k0), a.Tkv);
    a.Sq = min(q1 - q0, a.Sq);
    a.Skv = min(k1 - k0, a.Skv);
    a.coff = a.thd_bottom_right ? a.Skv - a.Sq : 0;
    a.q = static_cast<const T*>(a.q) + (int64_t)q0 * a.q_s[2];
    a.o = static_cast<T*>(a.o) + (int64_t)q0 * a.o_s[2];
    a.p = static_cast<T*>(a.p) + (int64_t)q0 * a.p_s[2];
    a.lse = a.lse + (int64_t)q0 * a.l_s[2];
    a.k = static_cast<const T*>(a.k) + (int64_t)k0 * a.k_s[2];
    a.v = static_cast<const T*>(a.v) + (int64_t)k0 * a.v_s[2];
}

template <bool USE_FIRST>
__device__ __forceinline__ const FwdArgs& pick_args(const FwdArgs& first, const FwdArgs& second) {
    if constexpr (USE_FIRST) return first;
    else return second;
}

// DROP: dropout with a caller keep-mask in sweep 2 (loader-wave kernels,
// whole calls): the stored probability is keep * P * drop_pscale and the
// output product takes keep * P * drop_oscale.
// THD: packed variable-length sequences (a workgroup rebased onto its
// sequence; the probability rows run to p_cols, zeros past the sequence's keys).
// HR: head rows (four-wave kernels without a loader wave, a.head_rows == 4):
// the compute waves take the query heads w.hq, w.hq + 1, ... of one KV group
// on the same 32 rows, sharing each K/V tile (and the head-shared mask rows)
// among the heads. CT: see TwoPassCfg (recorded tile classes of a bool mask
// that all query heads share).
template <typename T, int D, int NW, int MASK, bool VEC, int TN, bool NL, int SPL = 0, bool DROP = false,
          bool THD = false, bool HR = false, bool CT = false>
__global__ __attribute__((amdgpu_flat_work_group_size((NL ? NW : NW + 1) * 64, (NL ? NW : NW + 1) * 64),
                          amdgpu_waves_per_eu(NL ? 2 : SDPA_TP_WPE(NW))))
void sdpa_twopass_kernel(const FwdArgs a_in) {
    static_assert(SPL == 0 || !NL, "key ranges run on the loader-wave kernels");
    static_assert(!DROP || (SPL == 0 && !NL), "dropout runs on the whole-call loader-wave kernels");
    static_assert(!THD || (SPL == 0 && !NL && !DROP && MASK == MASK_NONE), "packed sequences: whole calls, no mask");
    static_assert(!HR || (NL && NW == 4 && SPL == 0 && !DROP && !THD), "head rows: four waves, no loader wave");
    static_assert(!CT || (NL && MASK == MASK_BOOL && VEC), "class records: no loader wave, a staged bool mask");
    using C = TwoPassCfg<T, D, NW, MASK, VEC, TN, NL, CT, HR>;
    static_assert(!CT || C::CT_FITS, "a mask tile must fit in a V buffer");
    static_assert(!NL || C::PSTAGE, "without a loader wave the probability stores must be staged");
    static_assert(C::LDS_BYTES <= 160 * 1024, "tile buffers exceed the 160 KB LDS of a compute unit");
    constexpr int BN = C::BN;
    constexpr int NKB = C::NKB;
    using TR = Tr<T>;
    using vec = typename TR::vec;
    constexpr int SZ = C::SZ;
    constexpr int KH = TR::KH;
    constexpr int KSTEP = 2 * KH;
    constexpr int NKS = D / KSTEP;           // MFMAs per 32x32 score block
    constexpr int QB = C::QB;
    constexpr int ND = D / 32;               // 32-wide head-dim chunks of O^T
    constexpr int ME = C::ME;

    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
    auto kbuf = [&](int b) -> uint8_t* { return smem + b * C::TILEB; };
    auto vbuf = [&](int b) -> uint8_t* { return smem + 2 * C::TILEB + b * C::TILEB; };
    auto mbuf = [&](int b) -> uint8_t* { return CT ? vbuf(b) : smem + 4 * C::TILEB + b * C::MTILEB; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
    const int n = lane & 31;
    const int hf = lane >> 5;

    const Work w = decode_block(SPL ? (int)blockIdx.x / a_in.n_splits : (int)blockIdx.x, a_in);
    FwdArgs seq_args;
    if constexpr (THD) {
        seq_args = a_in;
        thd_rebase<T>(seq_args, w.b);
        if (w.qblk * QB >= seq_args.Sq) return;  // past this sequence's queries (uniform)
    }
    const FwdArgs& a = pick_args<THD>(seq_args, a_in);
    const int pcols = THD ? a.p_cols : a.Skv;  // probability row length
    constexpr bool hrows = HR;
    const int hk = w.hq / a.group;
    const int q0 = hrows ? w.qblk * 32 : w.qblk * QB;
    const int kend = a.causal ? min(a.Skv, max(0, q0 + (hrows ? 32 : QB) + a.coff)) : a.Skv;
    const int ntiles = (kend + BN - 1) / BN;
    // this workgroup's tiles [t_lo, t_hi) (t_lo even: tile t stays in buffer t & 1)
    const int split = SPL ? (int)blockIdx.x % a.n_splits : 0;
    const int t_lo = SPL ? min(ntiles, split * a.split_tiles) : 0;
    const int t_hi = SPL ? min(ntiles, t_lo + a.split_tiles) : ntiles;

    const rsrc_t kr = make_rsrc(static_cast<const T*>(a.k) + w.b * a.k_s[0] + hk * a.k_s[1], a.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(a.v) + w.b * a.v_s[0] + hk * a.v_s[1], a.v_ext);
    rsrc_t mr = kr;
    if constexpr (MASK != MASK_NONE)
        mr = make_rsrc(static_cast<const uint8_t*>(a.mask) + (w.b * a.m_s[0] + w.hq * a.m_s[1]) * ME, a.m_ext);
    const uint32_t krow_bytes = (uint32_t)(a.k_s[2] * SZ);
    const uint32_t vrow_bytes = (uint32_t)(a.v_s[2] * SZ);

    // ------------------------------------------------ tile loads (buffer to LDS)
        // instruction j of a tile fills chunk positions [64 j, 64 j + 64), i.e.
        // rows j * RPI .. +RPI: lane l fetches the chunk the layout puts at
        // position 64 j + l
        // (j0, js): issue instructions j0, j0 + js, ... of the tile
        auto dma_k = [&](uint8_t* dst, int t, int j0, int js) SDPA_INLINE {
            const uint32_t so = (uint32_t)(t * BN) * krow_bytes;
#pragma unroll
            for (int j = 0; j < C::CPR * BN / 64; ++j) {
                if ((j - j0) % js != 0) continue;
                const int row = j * C::RPI + lane / C::CPR;
                const int chunk = (lane % C::CPR) ^ C::fk(row);
                const uint32_t vo = pred(t * BN + row < a.Skv, row * krow_bytes + (uint32_t)(chunk * 16));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(dst + j * 1024), 16, vo, so, 0, 0);
            }
        };
        auto dma_v = [&](uint8_t* dst, int t, int j0, int js) SDPA_INLINE {
            const uint32_t so = (uint32_t)(t * BN) * vrow_bytes;
#pragma unroll
            for (int j = 0; j < C::CPR * BN / 64; ++j) {
                if ((j - j0) % js != 0) continue;
                const int row = j * C::RPI + lane / C::CPR;
                const int chunk = (lane % C::CPR) ^ C::fv(row);
                const uint32_t vo = pred(t * BN + row < a.Skv, row * vrow_bytes + (uint32_t)(chunk * 16));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(dst + j * 1024), 16, vo, so, 0, 0);
            }
        };
        auto dma_m = [&](int t, int b, int j0, int js) SDPA_INLINE {
            if constexpr (C::MLDS) {
                const int mrow = lane / C::MCPR, mch = lane % C::MCPR;
#pragma unroll
                for (int j = 0; j < C::MNI; ++j) {
                    if ((j - j0) % js != 0) continue;
                    const int row = j * C::MRPI + mrow;  // query row q0 + row
                    // whole 16-byte chunks only: Skv is a multiple of the keys per chunk here
                    const uint32_t vo = pred((!hrows || row < 32) && q0 + row < a.Sq && t * BN + mch * (16 / ME) < a.Skv,
                                             (uint32_t)((int64_t)(q0 + row) * a.m_s[2] * ME) + (uint32_t)(mch * 16));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(mr, (lds_void*)(mbuf(b) + j * 1024), 16, vo,
                                                             (uint32_t)(t * BN * ME), 0, 0);
                }
            }
        };
    // ======================================================== loader wave
    if (!NL && wave == NW) {
        if constexpr (SPL != 2) {
            // sweep 1: K (+ mask)
            if (t_hi > t_lo) {
                dma_k(kbuf(0), t_lo, 0, 1);
                dma_m(t_lo, 0, 0, 1);
                wait_vmem();
            }
            __syncthreads();
            for (int t = t_lo; t < t_hi; ++t) {
                if (t + 1 < t_hi) {
                    dma_k(kbuf((t + 1) & 1), t + 1, 0, 1);
                    dma_m(t + 1, (t + 1) & 1, 0, 1);
                    wait_vmem();
                }
                __syncthreads();
            }
        }
        if constexpr (SPL != 1) {
            // sweep 2: K, V (+ mask)
            if (t_hi > t_lo) {
                dma_k(kbuf(0), t_lo, 0, 1);
                dma_v(vbuf(0), t_lo, 0, 1);
                dma_m(t_lo, 0, 0, 1);
                wait_vmem();
            }
            __syncthreads();
            for (int t = t_lo; t < t_hi; ++t) {
                if (t + 1 < t_hi) {
                    dma_k(kbuf((t + 1) & 1), t + 1, 0, 1);
                    dma_v(vbuf((t + 1) & 1), t + 1, 0, 1);
                    dma_m(t + 1, (t + 1) & 1, 0, 1);
                    wait_vmem();
                }
                __syncthreads();
            }
        }
        return;
    }

    // ======================================================== compute waves
    const int qw = hrows ? q0 : q0 + 32 * wave;
    const int hq_w = hrows ? w.hq + wave : w.hq;  // this wave's query head
    const int mrow0 = hrows ? 0 : 32 * wave;      // its rows in the staged mask tile
    const int qi = qw + n;
    const bool row_ok = qi < a.Sq;

    const rsrc_t qr = make_rsrc(static_cast<const T*>(a.q) + w.b * a.q_s[0] + hq_w * a.q_s[1], a.q_ext);
    const rsrc_t pr = make_rsrc(static_cast<T*>(a.p) + w.b * a.p_s[0] + hq_w * a.p_s[1], a.p_ext);
    const rsrc_t orr = make_rsrc(static_cast<T*>(a.o) + w.b * a.o_s[0] + hq_w * a.o_s[1], a.o_ext);
    const rsrc_t lr = make_rsrc(a.lse + w.b * a.l_s[0] + hq_w * a.l_s[1], a.l_ext);
    // byte offset of this lane's P row (past the descriptor when the row is out of range)
    const uint32_t prow = pred(row_ok, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.p_s[2] * SZ));

    // dropout keep bits of this lane's 16 keys of block kb: 1 keeps, 0 drops
    [[maybe_unused]] rsrc_t kpr = qr;
    [[maybe_unused]] uint32_t kp_row = 0;
    if constexpr (DROP) {
        kpr = make_rsrc(a.keep + w.b * a.kp_s[0] + hq_w * a.kp_s[1], a.kp_ext);
        kp_row = (uint32_t)((int64_t)(row_ok ? qi : 0) * a.kp_s[2]);
    }
    auto keep16 = [&](int k0, int kb, float* kv) SDPA_INLINE {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int j = k0 + 32 * kb + 16 * c + 8 * hf;
            if (a.keep_vec) {
                const u32x2 wv = ld64(kpr, pred(row_ok && j < a.Skv, kp_row + (uint32_t)j));
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[8 * c + e] = ((wv[e >> 2] >> (8 * (e & 3))) & 0xffu) ? 1.0f : 0.0f;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    kv[8 * c + e] = __builtin_amdgcn_raw_buffer_load_b8(
                                        kpr, pred(row_ok && j + e < a.Skv, kp_row + (uint32_t)((int64_t)(j + e) * a.kp_s[3])),
                                        0, 0) ? 1.0f : 0.0f;
            }
        }
    };

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

    // K operand (A) of S^T block kb, k-step c: lane (m, h) reads row 32kb +
    // swap23(m), elements c*KSTEP + h*KH .. +KH
    const int kr0 = swap23(n);
    auto k_operand = [&](const uint8_t* kt, int kb, int c) SDPA_INLINE -> vec {
        const int row = 32 * kb + kr0;
        const int elem = c * KSTEP + hf * KH;
        const uint8_t* p = kt + C::pos_k(row, elem * SZ / 16) * 16 + ((elem * SZ) & 15);
        if constexpr (sizeof(T) == 2) return as_vec<T>(*reinterpret_cast<const u32x4*>(p));
        else return *reinterpret_cast<const float*>(p);
    };
    // S^T of 32-key block kb (one MFMA chain over the head dim)
    // All K operand reads of the block are issued before its MFMA chain, so
    // the chain does not wait on LDS latency between steps.
    auto qk_block = [&](const uint8_t* kt, int kb) SDPA_INLINE -> f32x16 {
        f32x16 acc = {};
        vec ka[NKS];
#pragma unroll
        for (int c = 0; c < NKS; ++c) ka[c] = k_operand(kt, kb, c);
#pragma unroll
        for (int c = 0; c < NKS; ++c) acc = TR::mfma(ka[c], qf[c], acc);
        __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);  // the DS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, NKS, 0);  // then the MFMAs
        return acc;
    };

    // base-2 additive mask term of register r of block kb (a bool mask gives
    // 0 where it keeps the key, -inf where it removes it)
    auto mask_terms = [&](const uint8_t* mt, int k0, int kb, float* mv) SDPA_INLINE {
        if constexpr (MASK == MASK_NONE) {
            return;
        } else if constexpr (C::MLDS) {
            const uint8_t* base = mt + (mrow0 + n) * C::MROWB;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int jrel = 32 * kb + 16 * c + 8 * hf;
                if constexpr (ME == 1) {
                    const u32x2 wv = *reinterpret_cast<const u32x2*>(base + jrel);
#pragma unroll
                    for (int e = 0; e < 8; ++e) mv[8 * c + e] = ((wv[e >> 2] >> (8 * (e & 3))) & 0xffu) ? 0.0f : -INFINITY;
                } else if constexpr (ME == 2) {
                    const u32x4 wv = *reinterpret_cast<const u32x4*>(base + jrel * 2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) mv[8 * c + e] = Tr<T>::to_f((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu) * LOG2E;
                } else {
                    const u32x4 w0 = *reinterpret_cast<const u32x4*>(base + jrel * 4);
                    const u32x4 w1 = *reinterpret_cast<const u32x4*>(base + jrel * 4 + 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // element to a scalar first (bit_cast of a vector element reads element 0)
                        const uint32_t b0 = w0[e], b1 = w1[e];
                        mv[8 * c + e] = __builtin_bit_cast(float, b0) * LOG2E;
                        mv[8 * c + 4 + e] = __builtin_bit_cast(float, b1) * LOG2E;
                    }
                }
            }
        } else {
            // element-wise reads for layouts the staged path cannot take
            load_mask16<T, MASK, false>(a, mr, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.m_s[2] * ME), k0 + 32 * kb,
                                        hf, mv);
        }
    };

    // What the staged bool mask tile does to this wave's 32 rows: DEAD, it
    // removes every key (a key-padding tail, for instance): the tile adds
    // nothing to the row sums and its probabilities are all zero, so its
    // products and exponentials are skipped (the same bits as computing
    // them); FULL, it keeps every key: the tile takes the unmasked code (the
    // scale folded into one fma per exponent, one rounding fewer).
    constexpr int TILE_DEAD = 1, TILE_FULL = 2;
    auto tile_flags = [&](const uint8_t* mt) SDPA_INLINE -> int {
        if constexpr (MASK == MASK_BOOL && C::MLDS) {
            constexpr int NCH = 32 * C::MROWB / 16 / 64;  // 16-byte chunks per lane
            static_assert(NCH >= 1 && 32 * C::MROWB % 1024 == 0, "mask tile rows of a wave must split into lane chunks");
            const u32x4* c = reinterpret_cast<const u32x4*>(mt + mrow0 * C::MROWB) + lane * NCH;
            uint32_t any = 0u, zero_byte = 0u;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const u32x4 x = c[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = x[e];
                    any |= w;
                    zero_byte |= (w - 0x01010101u) & ~w & 0x80808080u;  // nonzero iff w has a zero byte
                }
            }
            const bool dead = __builtin_amdgcn_ballot_w64(any != 0u) == 0;
            const bool full = __builtin_amdgcn_ballot_w64(zero_byte != 0u) == 0;
            return (dead ? TILE_DEAD : 0) | (full ? TILE_FULL : 0);
        } else {
            return 0;
        }
    };
    // CT: the classes sweep 1 found for this wave's rows, 2 bits per tile,
    // tile t in lane t / 16 (up to 1024 tiles); with head rows the same in
    // every wave of the workgroup (its waves share the rows)
    uint32_t cls_rec = 0u;
    auto record_flags = [&](int t, int flags) SDPA_INLINE {
        if constexpr (CT) cls_rec |= lane == (t >> 4) ? (uint32_t)flags << (2 * (t & 15)) : 0u;
    };
    auto recorded_flags = [&](int t) SDPA_INLINE -> int {
        return (int)(((uint32_t)__builtin_amdgcn_readlane((int)cls_rec, t >> 4) >> (2 * (t & 15))) & 3u);
    };

    // Base-2 scaled, masked scores t[r] of one block. `edge`: the block may
    // hold keys past Skv or past this wave's causal diagonal.
    auto scores = [&](const f32x16& acc, const float* mv, int kb, int k0, bool edge, float* t) SDPA_INLINE {
        const int jb = k0 + 32 * kb;
        // register r holds key jb + kk(hf, r) = jb + 8 hf + kk(0, r); it is
        // dropped when kk(0, r) > lim (a compile-time constant per register)
        const int lim = edge ? min(a.Skv - 1 - jb, a.causal ? qi + a.coff - jb : 0x7fffffff) - 8 * hf : 0x7fffffff;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // fma with a 0 term rounds like the plain product
            const float x = MASK != MASK_NONE ? __builtin_fmaf(acc[r], a.scale_log2, mv[r]) : acc[r] * a.scale_log2;
            bool drop = false;
            if (edge) drop = kk(0, r) > lim;
            t[r] = drop ? -INFINITY : x;
        }
    };

    // Tiles of this wave: [0, t_fast) hold only keys every row keeps (no
    // edge), [t_fast, t_comp) reach past Skv or the causal diagonal, and
    // [t_comp, ntiles) lie wholly above the diagonal. Each range has its own
    // loop, so each loop body is straight-line code; every wave still meets
    // one barrier per tile, as the loader wave does.
    // a wave whose rows all lie past Sq (the last block of a ragged Sq) only
    // keeps the barrier count
    const bool live = qw < a.Sq;
    const int dlast = qw + 31 + a.coff;  // causal: last key the wave's last row keeps
    const int t_comp = !live ? 0 : a.causal ? (dlast < 0 ? 0 : min(ntiles, dlast / BN + 1)) : ntiles;
    const int t_fast = min(t_comp, a.causal ? min(a.Skv / BN, max(0, qw + a.coff + 1) / BN) : a.Skv / BN);
    // the same split within this workgroup's tiles
    const int tf = min(max(t_fast, t_lo), t_hi);
    const int tc = min(max(t_comp, t_lo), t_hi);

    // ---------------- sweep 1: row maximum and sum (base 2)
    float m_run = -INFINITY, l_run = 0.0f;
    auto sweep1_tile = [&](int t, auto edge_c) SDPA_INLINE {
        constexpr bool edge = decltype(edge_c)::value;
        const int k0 = t * BN;
        const int buf = t & 1;
        const int flags = tile_flags(mbuf(buf));
        record_flags(t, flags);
        if (flags & TILE_DEAD) return;
        const bool plain = MASK == MASK_NONE || (flags & TILE_FULL);  // no key of the tile is masked
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const f32x16 acc = qk_block(kbuf(buf), kb);
            float sum = 0.0f;
            if (plain && !edge && a.scale_log2 > 0.0f) {
                // max on the raw scores (the scale is positive), then one fma per exponent
                float mx = acc[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
                const float mn = fmaxf(m_run, mx * a.scale_log2);
#pragma unroll
                for (int r = 0; r < 16; ++r) sum += fast_exp2(__builtin_fmaf(acc[r], a.scale_log2, -mn));
                l_run = l_run * fast_exp2(m_run - mn) + sum;
                m_run = mn;
            } else {
                float mv[16];
                mask_terms(mbuf(buf), k0, kb, mv);
                float tt[16];
                scores(acc, mv, kb, k0, edge, tt);
                float mt = tt[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mt = fmaxf(mt, tt[r]);
                const float mn = fmaxf(m_run, mt);
                if (mn != -INFINITY) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sum += fast_exp2(tt[r] - mn);
                    l_run = l_run * fast_exp2(m_run - mn) + sum;
                    m_run = mn;
                }
            }
        }
    };
    // Without a loader wave each compute wave issues its share of the next
    // tile's loads before working on the current one, and waits for them
    // (its only outstanding memory operations here) before the barrier.
    auto load1 = [&](int t) SDPA_INLINE {
        if constexpr (NL) {
            if (t < ntiles) {
                dma_k(kbuf(t & 1), t, wave, NW);
                dma_m(t, t & 1, wave, NW);
            }
        }
    };
    auto end_tile = [&]() SDPA_INLINE {
        if constexpr (NL) wait_vmem();
        __syncthreads();  // tile t consumed, tile t+1 staged
    };
    // Fast tiles without a mask, software-pipelined: the MFMA chain of the
    // next score block is interleaved with the max / exp2 / sum fold of the
    // previous one, so a single wave keeps the matrix unit and the vector
    // unit busy together. The fold of a tile's last block runs after the
    // tile barrier (its scores are in registers). Same arithmetic, in the
    // same order, as sweep1_tile's fast branch.
    auto fold_fast = [&](const f32x16& acc) SDPA_INLINE {
        float mx = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        const float mn = fmaxf(m_run, mx * a.scale_log2);
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(__builtin_fmaf(acc[r], a.scale_log2, -mn));
        l_run = l_run * fast_exp2(m_run - mn) + sum;
        m_run = mn;
    };
    // S^T of block kb of tile buffer kt, with the fold of `prev` interleaved
    // by hand (scheduling fences keep the order): the DS reads, the fold's
    // max while they land, then per MFMA step the exp2 / sum of a few
    // scores. The sum runs over r in order, as in fold_fast.
    auto qk_fold = [&](const uint8_t* kt, int kb, const f32x16& prev) SDPA_INLINE -> f32x16 {
        f32x16 acc = {};
        vec ka[NKS];
#pragma unroll
        for (int c = 0; c < NKS; ++c) ka[c] = k_operand(kt, kb, c);
        __builtin_amdgcn_sched_barrier(0);
        float mx = prev[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, prev[r]);
        const float mn = fmaxf(m_run, mx * a.scale_log2);
        const float resc = fast_exp2(m_run - mn);
        float sum = 0.0f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            acc = TR::mfma(ka[c], qf[c], acc);
#pragma unroll
            for (int e = c * 16 / NKS; e < (c + 1) * 16 / NKS; ++e)
                sum += fast_exp2(__builtin_fmaf(prev[e], a.scale_log2, -mn));
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run = l_run * resc + sum;
        m_run = mn;
        return acc;
    };
    const bool pipe1 = MASK == MASK_NONE && a.scale_log2 > 0.0f;

    if constexpr (SPL != 2) {
    load1(t_lo);
    end_tile();  // tile t_lo staged
    {
        int t = t_lo;
        if (pipe1 && tf > t_lo) {
            load1(t_lo + 1);
            f32x16 pend = qk_block(kbuf(0), 0);
#pragma unroll
            for (int kb = 1; kb < NKB; ++kb) pend = qk_fold(kbuf(0), kb, pend);
            end_tile();
            // tiles in pairs, so that each one's buffer is a compile-time
            // constant (its offset folds into the LDS instructions)
            auto fast1 = [&](int tt, auto par) SDPA_INLINE {
                load1(tt + 1);
                const uint8_t* kt = kbuf(decltype(par)::value);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) pend = qk_fold(kt, kb, pend);
                end_tile();
            };
            for (t = t_lo + 1; t + 1 < tf; t += 2) {
                fast1(t, std::integral_constant<int, 1>{});
                fast1(t + 1, std::integral_constant<int, 0>{});
            }
            if (t < tf) fast1(t++, std::integral_constant<int, 1>{});
            fold_fast(pend);
        }
        for (; t < tf; ++t) {
            load1(t + 1);
            sweep1_tile(t, std::false_type{});
            end_tile();
        }
        for (; t < tc; ++t) {
            load1(t + 1);
            sweep1_tile(t, std::true_type{});
            end_tile();
        }
        for (; t < t_hi; ++t) {
            load1(t + 1);
            end_tile();
        }
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
    }
    // row index of this lane in the key-range workspace
    const int64_t ws_row = ((int64_t)split * a.B * a.Hq + (int64_t)w.b * a.Hq + w.hq) * a.Sq + (row_ok ? qi : 0);
    if constexpr (SPL == 1) {  // this range's (max, sum) of each row, base 2
        if (row_ok && hf == 0) a.ws_ml[ws_row] = float2{m_run, l_run};
        return;
    }
    if constexpr (SPL == 2) {  // fold every range's statistics, in range order (the same bits in each range)
        const int64_t stride = (int64_t)a.B * a.Hq * a.Sq;
        const int64_t r0 = ws_row - (int64_t)split * stride;
        m_run = -INFINITY;
        l_run = 0.0f;
        for (int s2 = 0; s2 < a.n_splits; ++s2) {
            const float2 st = row_ok ? a.ws_ml[r0 + s2 * stride] : float2{-INFINITY, 0.0f};
            const float mn = fmaxf(m_run, st.x);
            if (mn != -INFINITY) {
                l_run = l_run * fast_exp2(m_run - mn) + st.y * fast_exp2(st.x - mn);
                m_run = mn;
            }
        }
    }
    const bool dead = (m_run == -INFINITY);
    // dead rows: lse2 = +inf makes every probability exp2(-inf) = +0
    const float lse2 = dead ? INFINITY : m_run + __log2f(l_run);

    // ---------------- sweep 2: P = exp2(t - lse2), store, O^T += V^T P^T
    f32x16 oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};

    // Transposing-read address for the V^T operand: as source lane s = lane %
    // 16 of group g = lane / 16 this lane reads 4 head-dim columns of key row
    // 8(g/2) + s/4 (+ 4 for the second read); the column group is permuted
    // (bits 0 and 1 of s exchanged) so that output lane i receives head-dim
    // column swap23(i) of its half of a 32-wide chunk.
    const int trg = lane >> 4, trs = lane & 15;
    const int tr_sig = ((trs & 1) << 1) | ((trs >> 1) & 1);
    const int tr_row = 8 * (trg >> 1) + (trs >> 2);
    const int tr_col = 16 * (trg & 1) + 4 * tr_sig;
    auto v_operand = [&](const uint8_t* vt, int key0, int d) SDPA_INLINE -> vec {
        if constexpr (sizeof(T) == 2) {
            // rows key0 + tr_row and key0 + tr_row + 4, columns 32d + tr_col .. +3
            u32x2 half[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int row = key0 + tr_row + 4 * r;
                const int col = 32 * d + tr_col;
                half[r] = lds_read_tr16(vt + C::pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
            }
            return __builtin_bit_cast(vec, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
        } else {
            return vec{};
        }
    };

    // store of 8 probabilities (one run) of block kb, run c
    auto store_run = [&](int k0, int kb, int c, bool edge, const float* x) SDPA_INLINE {
        const int jrel = 32 * kb + 16 * c + 8 * hf;
        if constexpr (VEC) {
            uint32_t vo = prow + (uint32_t)(jrel * SZ);
            if (edge) vo = pred(k0 + jrel < pcols, vo);
            if constexpr (sizeof(T) == 2) {
                st128s(pr, vo, (uint32_t)(k0 * SZ), __builtin_bit_cast(u32x4, Tr<T>::cvt8(x)));
            } else {
                st128s(pr, vo, (uint32_t)(k0 * SZ),
                       u32x4{__builtin_bit_cast(uint32_t, x[0]), __builtin_bit_cast(uint32_t, x[1]),
                             __builtin_bit_cast(uint32_t, x[2]), __builtin_bit_cast(uint32_t, x[3])});
                st128s(pr, vo == OOB ? OOB : vo + 16, (uint32_t)(k0 * SZ),
                       u32x4{__builtin_bit_cast(uint32_t, x[4]), __builtin_bit_cast(uint32_t, x[5]),
                             __builtin_bit_cast(uint32_t, x[6]), __builtin_bit_cast(uint32_t, x[7])});
            }
        } else {
            store8<T, false>(pr, row_ok ? prow : 0u, row_ok, k0 + jrel, pcols, x);
        }
    };

    uint8_t* pst = smem + C::KVM_BYTES + (C::PSTAGE ? wave * C::PSTB : 0);  // this wave's staged P tile
    // whole-row stores of the staged P tile with first key k0
    auto store_staged = [&](int k0, bool edge) SDPA_INLINE {
#pragma unroll
        for (int i = 0; i < 32 * C::ZC / 64; ++i) {
            const int row = i * (64 / C::ZC) + lane / C::ZC;
            const int chunk = lane % C::ZC;
            const u32x4 bits = *reinterpret_cast<const u32x4*>(pst + C::pos_p(row, chunk) * 16);
            const int grow = qw + row, key = k0 + chunk * (16 / SZ);
            const bool ok = grow < a.Sq && (!edge || key < pcols);
            st128_nt(pr, pred(ok, (uint32_t)((int64_t)(grow < a.Sq ? grow : 0) * a.p_s[2] * SZ) + (uint32_t)(key * SZ)),
                  bits);
        }
    };
    // a tile wholly above this wave's diagonal: P is zero
    auto zero_tile = [&](int t) SDPA_INLINE {
        if (!live) {
            // nothing to store
        } else if constexpr (VEC) {
            // whole-row 16-byte stores: instruction i covers rows 64 i / ZC ..
            constexpr int ZC = BN * SZ / 16;  // 16-byte chunks per row of the tile
#pragma unroll
            for (int i = 0; i < 32 * ZC / 64; ++i) {
                const int row = qw + i * (64 / ZC) + lane / ZC;
                const int key = t * BN + (lane % ZC) * (16 / SZ);
                st128_nt(pr, pred(row < a.Sq && key < pcols,
                               (uint32_t)((int64_t)(row < a.Sq ? row : 0) * a.p_s[2] * SZ) + (uint32_t)(key * SZ)),
                      u32x4{0u, 0u, 0u, 0u});
            }
        } else {
            const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const bool edge = (t + 1) * BN > pcols;
#pragma unroll
            for (int q = 0; q < 2 * NKB; ++q) store_run(t * BN, q >> 1, q & 1, edge, z);
        }
    };
    // buf: t & 1, passed as a constant by the paired fast loop
    auto sweep2_tile = [&](int t, auto edge_c, int buf) SDPA_INLINE {
        constexpr bool edge = decltype(edge_c)::value;
        const int k0 = t * BN;
        const int flags = CT ? recorded_flags(t) : tile_flags(mbuf(buf));
        const bool plain = MASK == MASK_NONE || (flags & TILE_FULL);  // no key of the tile is masked
        if (flags & TILE_DEAD) {  // P = 0, O unchanged
            if constexpr (C::PSTAGE) {
#pragma unroll
                for (int i = 0; i < C::PSTB / 1024; ++i)
                    *reinterpret_cast<u32x4*>(pst + (i * 64 + lane) * 16) = u32x4{0u, 0u, 0u, 0u};
                if constexpr (!NL) store_staged(k0, edge);
            } else {
                zero_tile(t);
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const f32x16 acc = qk_block(kbuf(buf), kb);
            float p[16];
            if (plain && !edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(acc[r], a.scale_log2, -lse2));
            } else {
                float mv[16];
                if constexpr (CT)  // mixed tiles only: the mask from memory
                    load_mask16<T, MASK, true>(a, mr, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.m_s[2] * ME),
                                               k0 + 32 * kb, hf, mv);
                else
                    mask_terms(mbuf(buf), k0, kb, mv);
                float tt[16];
                scores(acc, mv, kb, k0, edge, tt);
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = fast_exp2(tt[r] - lse2);
            }
            // dropout: ps = what is stored, p = what the output product takes
            [[maybe_unused]] float ps[16];
            if constexpr (DROP) {
                float kv[16];
                keep16(k0, kb, kv);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pd = p[r] * kv[r];
                    ps[r] = pd * a.drop_pscale;
                    p[r] = pd * a.drop_oscale;
                }
            }
            if constexpr (sizeof(T) == 2) {
                vec va[2][ND];  // V^T operands of both 16-key halves, read ahead of the MFMAs
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                    for (int d = 0; d < ND; ++d) va[c2][d] = v_operand(vbuf(buf), 32 * kb + 16 * c2, d);
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    // the rounded probabilities (stored) and their rounded
                    // residual: O accumulates P to twice the dtype's precision
                    const vec pv = TR::cvt8(p + 8 * c2);
                    const vec pl = TR::lo8(p + 8 * c2, pv);
                    const float* stored = DROP ? ps + 8 * c2 : p + 8 * c2;
                    if constexpr (C::PSTAGE) {
                        const int chunk = (32 * kb + 16 * c2 + 8 * hf) * SZ / 16;
                        *reinterpret_cast<u32x4*>(pst + C::pos_p(n, chunk) * 16) =
                            __builtin_bit_cast(u32x4, DROP ? TR::cvt8(stored) : pv);
                    } else {
                        store_run(k0, kb, c2, edge, stored);
                    }
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[c2][d], pv, oacc[d]);
#pragma unroll
                    for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va[c2][d], pl, oacc[d]);
                }
            } else {
                const float* stored = DROP ? ps : p;
                if constexpr (C::PSTAGE) {
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const int chunk = (32 * kb + 16 * c2 + 8 * hf) * SZ / 16 + h2;
                            const float* x = stored + 8 * c2 + 4 * h2;
                            *reinterpret_cast<u32x4*>(pst + C::pos_p(n, chunk) * 16) =
                                u32x4{__builtin_bit_cast(uint32_t, x[0]), __builtin_bit_cast(uint32_t, x[1]),
                                      __builtin_bit_cast(uint32_t, x[2]), __builtin_bit_cast(uint32_t, x[3])};
                        }
                } else {
                    store_run(k0, kb, 0, edge, stored);
                    store_run(k0, kb, 1, edge, stored + 8);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * kb + kk(hf, r);
#pragma unroll
                    for (int d = 0; d < ND; ++d) {
                        const int col = 32 * d + swap23(n);
                        const float va = *reinterpret_cast<const float*>(
                            vbuf(buf) + C::pos_v(row, col * SZ / 16) * 16 + ((col * SZ) & 15));
                        oacc[d] = TR::mfma(va, p[r], oacc[d]);
                    }
                }
            }
        }
        if constexpr (C::PSTAGE && !NL) store_staged(k0, edge);
    };
    // Fast tile (no mask, no edge, 16-bit, two 32-key blocks, staged P) with
    // the two blocks software-pipelined by hand (scheduling fences keep the
    // order): block 1's S^T chain runs under block 0's exp2, block 0's
    // O^T += V^T P^T chain under block 1's exp2, and the operand reads go out
    // under the MFMAs. Same arithmetic, and the same accumulation order into
    // O^T, as sweep2_tile.
    auto sweep2_pipe = [&](int t, int buf) SDPA_INLINE {
      if constexpr (sizeof(T) == 2 && NKB == 2) {
        const uint8_t* kt = kbuf(buf);
        const uint8_t* vt = vbuf(buf);
        vec ka[NKS], kn[NKS];
        vec va0[2][ND], va1[2][ND];
#pragma unroll
        for (int c = 0; c < NKS; ++c) ka[c] = k_operand(kt, 0, c);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 acc0 = {};
#pragma unroll
        for (int c = 0; c < NKS; ++c) {  // S^T of block 0; reads of block 1's K and block 0's V
            acc0 = TR::mfma(ka[c], qf[c], acc0);
            kn[c] = k_operand(kt, 1, c);
            va0[c / ND][c % ND] = v_operand(vt, 16 * (c / ND), c % ND);  // 2 ND = NKS operands
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x16 acc1 = {};
        float p0[16], p1[16];
#pragma unroll
        for (int c = 0; c < NKS; ++c) {  // S^T of block 1 under block 0's exp2
            acc1 = TR::mfma(kn[c], qf[c], acc1);
#pragma unroll
            for (int e = c * 16 / NKS; e < (c + 1) * 16 / NKS; ++e)
                p0[e] = fast_exp2(__builtin_fmaf(acc0[e], a.scale_log2, -lse2));
            __builtin_amdgcn_sched_barrier(0);
        }
        vec pv0[2], pv1[2], pl0[2], pl1[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            pv0[c2] = TR::cvt8(p0 + 8 * c2);
            pl0[c2] = TR::lo8(p0 + 8 * c2, pv0[c2]);
            *reinterpret_cast<u32x4*>(pst + C::pos_p(n, (16 * c2 + 8 * hf) * SZ / 16) * 16) =
                __builtin_bit_cast(u32x4, pv0[c2]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T (P_hi + P_lo)^T of block 0 under block 1's exp2, in the
        // order of sweep2_tile: per 16-key half, the hi products then the lo
#pragma unroll
        for (int i = 0; i < 4 * ND; ++i) {
            const int c2 = i / (2 * ND), part = (i / ND) & 1, d = i % ND;
            oacc[d] = TR::mfma(va0[c2][d], part ? pl0[c2] : pv0[c2], oacc[d]);
            if (part == 0) va1[c2][d] = v_operand(vt, 32 + 16 * c2, d);
#pragma unroll
            for (int e = i * 16 / (4 * ND); e < (i + 1) * 16 / (4 * ND); ++e)
                p1[e] = fast_exp2(__builtin_fmaf(acc1[e], a.scale_log2, -lse2));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            pv1[c2] = TR::cvt8(p1 + 8 * c2);
            pl1[c2] = TR::lo8(p1 + 8 * c2, pv1[c2]);
            *reinterpret_cast<u32x4*>(pst + C::pos_p(n, (32 + 16 * c2 + 8 * hf) * SZ / 16) * 16) =
                __builtin_bit_cast(u32x4, pv1[c2]);
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
            for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va1[c2][d], pv1[c2], oacc[d]);
#pragma unroll
            for (int d = 0; d < ND; ++d) oacc[d] = TR::mfma(va1[c2][d], pl1[c2], oacc[d]);
        }
        if constexpr (!NL) store_staged(t * BN, false);
      }
    };
    // (not without a loader wave: its deferred stores leave too few registers)
    constexpr bool PIPE2 = sizeof(T) == 2 && NKB == 2 && MASK == MASK_NONE && C::PSTAGE && !NL && !DROP;
    // Without a loader wave a tile's probability stores are issued at the
    // start of the next tile (from the staged copy), so the wait before the
    // next barrier finds them a whole tile old rather than just issued.
    auto load2 = [&](int t) SDPA_INLINE {
        if constexpr (NL) {
            // CT: no mask tiles; with head rows no K/V for a tile every row
            // of the workgroup drops (its classes are the same in every wave)
            if (t < ntiles && !(CT && HR && (recorded_flags(t) & TILE_DEAD))) {
                dma_k(kbuf(t & 1), t, wave, NW);
                dma_v(vbuf(t & 1), t, wave, NW);
                if constexpr (!CT) dma_m(t, t & 1, wave, NW);
            }
        }
    };
    int pend_k0 = -1;          // key of the staged tile not yet stored (NL)
    bool pend_edge = false;
    auto flush = [&]() SDPA_INLINE {
        if constexpr (NL) {
            if (pend_k0 >= 0) store_staged(pend_k0, pend_edge);
            pend_k0 = -1;
        }
    };
    load2(t_lo);
    end_tile();  // tile t_lo staged
    {
        int t = t_lo;
        auto fast2 = [&](int tt, int buf) SDPA_INLINE {
            flush();
            load2(tt + 1);
            if constexpr (PIPE2) sweep2_pipe(tt, buf);
            else sweep2_tile(tt, std::false_type{}, buf);
            pend_k0 = tt * BN;
            pend_edge = false;
            end_tile();
        };
        for (; t + 1 < tf; t += 2) {  // in pairs: constant buffers, as in sweep 1
            fast2(t, 0);
            fast2(t + 1, 1);
        }
        if (t < tf) fast2(t++, 0);
        for (; t < tc; ++t) {
            flush();
            load2(t + 1);
            sweep2_tile(t, std::true_type{}, t & 1);
            pend_k0 = t * BN;
            pend_edge = true;
            end_tile();
        }
        flush();
        // whole tiles above this wave's diagonal: P is zero, O unchanged
        // (without a loader wave the zeros are written after the last tile)
        const int t_zero = t;
        for (; t < t_hi; ++t) {
            load2(t + 1);
            if constexpr (!NL) zero_tile(t);
            end_tile();
        }
        if constexpr (NL)
            for (int tz = t_zero; tz < t_hi; ++tz) zero_tile(tz);
    }

    // ---------------- O: lane (n, h) holds O[qi][32d + 8h ..+8) and [32d + 16 + 8h ..+8)
    if constexpr (SPL == 2) {  // float32 partial O of this key range
        float* const orow = a.ws_o + ws_row * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e4 = 0; e4 < 2; ++e4)
                    if (row_ok)
                        *reinterpret_cast<f32x4*>(orow + 32 * d + 16 * h2 + 8 * hf + 4 * e4) =
                            f32x4{oacc[d][8 * h2 + 4 * e4], oacc[d][8 * h2 + 4 * e4 + 1], oacc[d][8 * h2 + 4 * e4 + 2],
                                  oacc[d][8 * h2 + 4 * e4 + 3]};
    } else {
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
    // (with key ranges: written by the last range; LSE by the first)
    if (SPL == 0 || split == a.n_splits - 1) zero_rows<T, VEC>(pr, a.p_s[2], qw, a.Sq, ntiles * BN, pcols, lane);
    if (SPL == 0 || split == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dead ? -INFINITY : lse2 * LN2), lr,
                                              pred(row_ok && hf == 0, (uint32_t)((int64_t)(row_ok ? qi : 0) * a.l_s[2] * 4)),
                                              0, 0);
}

// Keys per tile by mask kind: 32 with a bool mask, 64 otherwise. A bool mask
// tile of 32 keys is more often wholly kept or wholly removed for a wave's
// rows (key padding), which skips its decode or its arithmetic: the GQA
// key-padding workload runs 166 -> 153 us (MI355X); without a mask or with an
// additive one, 32-key tiles are slower (2k causal prefill 90 -> 119 us,
// decode with an additive mask 32 -> 40 us).
template <int MK>
constexpr int tile_keys() { return MK == MASK_BOOL ? 32 : 64; }

// Packed variable-length sequences: two compute waves and a loader wave, no mask.
template <typename T, int D, bool VEC>
static int launch_twopass_thd(const FwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, 2, MASK_NONE, VEC, tile_keys<MASK_NONE>(), false, 0, false, true>),
                       dim3(a.n_blocks), dim3(3 * 64), 0, s, a);
    return (int)hipGetLastError();
}

template <typename T, int D, int NW, bool VEC, bool NL, bool DROP = false>
static int launch_twopass_mask(int mask_kind, const FwdArgs& a, hipStream_t s) {
    dim3 grid(a.n_blocks), block((NL ? NW : NW + 1) * 64);
    switch (mask_kind) {
#define SDPA_TP_CASE(MK)                                                                                          \
    case MK:                                                                                                      \
        if constexpr (!NL || TwoPassCfg<T, D, NW, MK, VEC, tile_keys<MK>(), true>::PSTAGE) {                       \
            if (a.head_rows > 0) {                                                                                \
                if constexpr (NL && NW == 4 && !DROP && MK == MASK_BOOL && VEC &&                                 \
                              TwoPassCfg<T, D, NW, MK, VEC, 64, true, true, true>::PSTAGE) {                        \
                    if (a.Skv <= 64 * 1024) {                                                                     \
                        hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MK, VEC, 64, NL, 0, false, false, true, \
                                                                true>), grid, block, 0, s, a);                    \
                        break;                                                                                    \
                    }                                                                                             \
                }                                                                                                 \
                if constexpr (NL && NW == 4 && !DROP) {                                                           \
                    hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MK, VEC, tile_keys<MK>(), NL, 0, false, false, \
                                                            true>), grid, block, 0, s, a);                        \
                    break;                                                                                        \
                } else {                                                                                          \
                    return (int)hipErrorInvalidValue;                                                             \
                }                                                                                                 \
            }                                                                                                     \
            if constexpr (NL && NW == 4 && !DROP && MK == MASK_BOOL && VEC &&                                     \
                          TwoPassCfg<T, D, NW, MK, VEC, 64, true, true>::PSTAGE &&                                  \
                          TwoPassCfg<T, D, NW, MK, VEC, 64, true, true>::CT_FITS) {                                 \
                if (a.m_s[1] == 0 && a.Skv <= 64 * 1024) { /* a mask all query heads share */                   \
                    hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MK, VEC, 64, NL, 0, false, false, false, true>), \
                                       grid, block, 0, s, a);                                                     \
                    break;                                                                                        \
                }                                                                                                 \
            }                                                                                                     \
            hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, NW, MK, VEC, tile_keys<MK>(), NL, 0, DROP>), grid, block, \
                               0, s, a);                                                                          \
            break;                                                                                                \
        } else {                                                                                      \
            return (int)hipErrorInvalidValue;                                                         \
        }
        SDPA_TP_CASE(MASK_NONE)
        SDPA_TP_CASE(MASK_BOOL)
        SDPA_TP_CASE(MASK_ADD)
#undef SDPA_TP_CASE
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// Output of a call split into key ranges: the ranges' float32 partial O of
// each row summed in range order and rounded once to the output dtype. One
// thread per 8 consecutive columns of a row (16-byte aligned output rows).
template <typename T>
__global__ __launch_bounds__(256) void sdpa_split_combine_kernel(const FwdArgs a, int D) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    const int cpr = D / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * cpr) return;
    const int64_t row = i / cpr;
    const int c = (int)(i - row * cpr) * 8;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < a.n_splits; ++s2) {
        const float* src = a.ws_o + ((int64_t)s2 * rows + row) * D + c;
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] += u0[e];
            x[4 + e] += u1[e];
        }
    }
    const int q = (int)(row % a.Sq);
    const int64_t bh = row / a.Sq;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    T* o = static_cast<T*>(a.o) + b * a.o_s[0] + h * a.o_s[1] + (int64_t)q * a.o_s[2] + c;
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(o) = __builtin_bit_cast(u32x4, Tr<T>::cvt8(x));
    } else {
        *reinterpret_cast<f32x4*>(o) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
}

// A call split into key ranges (two compute waves and a loader wave,
// 16-byte layouts): statistics launch, probability launch, output combine.
template <typename T, int D>
static int launch_twopass_split(int mask_kind, const FwdArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_blocks * (unsigned)a.n_splits), block(3 * 64);
    switch (mask_kind) {
#define SDPA_SPLIT_CASE(MK)                                                                                      \
    case MK:                                                                                                     \
        hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, 2, MK, true, tile_keys<MK>(), false, 1>), grid, block, 0, s, a); \
        hipLaunchKernelGGL((sdpa_twopass_kernel<T, D, 2, MK, true, tile_keys<MK>(), false, 2>), grid, block, 0, s, a); \
        break;
        SDPA_SPLIT_CASE(MASK_NONE)
        SDPA_SPLIT_CASE(MASK_BOOL)
        SDPA_SPLIT_CASE(MASK_ADD)
#undef SDPA_SPLIT_CASE
        default: return (int)hipErrorInvalidValue;
    }
    const int64_t n = (int64_t)a.B * a.Hq * a.Sq * (D / 8);
    hipLaunchKernelGGL(sdpa_split_combine_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, D);
    return (int)hipGetLastError();
}

// Whether four compute waves without a loader wave can run for this shape:
// the staged probability tiles of four waves must fit next to the K/V (and
// mask) tiles within the LDS of half a CU.
template <typename T>
static bool twopass_nl_ok_t(int D, int mask_kind) {
#define SDPA_NL(DD, MK) TwoPassCfg<T, DD, 4, MK, true, tile_keys<MK>(), true>::PSTAGE
#define SDPA_NL_D(DD)                                                                 \
    case DD:                                                                          \
        return mask_kind == MASK_NONE ? SDPA_NL(DD, MASK_NONE)                        \
             : mask_kind == MASK_BOOL ? SDPA_NL(DD, MASK_BOOL) : SDPA_NL(DD, MASK_ADD);
    switch (D) {
        SDPA_NL_D(32)
        SDPA_NL_D(64)
        SDPA_NL_D(128)
        default: return false;
    }
#undef SDPA_NL_D
#undef SDPA_NL
}

// waves: 4 = four compute waves without a loader wave (16-byte layouts only,
// when twopass_nl_ok); 3 or 2 = that many compute waves plus a loader wave.
// Element-wise layouts only need correctness: they get one two-wave shape.
// float32 takes at most two compute waves at D = 128 (its tiles are twice
// as large: two waves keep them within LDS).
template <typename T>
static int launch_twopass_t(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (a.thd) {  // packed sequences: two compute waves and a loader wave, no mask, whole calls
        if (waves != 2 || a.n_splits > 1 || drop || mask_kind != MASK_NONE) return (int)hipErrorInvalidValue;
        switch (D) {
            case 32: return vec ? launch_twopass_thd<T, 32, true>(a, s) : launch_twopass_thd<T, 32, false>(a, s);
            case 64: return vec ? launch_twopass_thd<T, 64, true>(a, s) : launch_twopass_thd<T, 64, false>(a, s);
            case 128: return vec ? launch_twopass_thd<T, 128, true>(a, s) : launch_twopass_thd<T, 128, false>(a, s);
            default: return (int)hipErrorInvalidValue;
        }
    }
    if (drop) {  // dropout: two compute waves and a loader wave, whole calls
        if (waves != 2 || a.n_splits > 1) return (int)hipErrorInvalidValue;
        switch (D) {
            case 32: return vec ? launch_twopass_mask<T, 32, 2, true, false, true>(mask_kind, a, s)
                                : launch_twopass_mask<T, 32, 2, false, false, true>(mask_kind, a, s);
            case 64: return vec ? launch_twopass_mask<T, 64, 2, true, false, true>(mask_kind, a, s)
                                : launch_twopass_mask<T, 64, 2, false, false, true>(mask_kind, a, s);
            case 128: return vec ? launch_twopass_mask<T, 128, 2, true, false, true>(mask_kind, a, s)
                                 : launch_twopass_mask<T, 128, 2, false, false, true>(mask_kind, a, s);
            default: return (int)hipErrorInvalidValue;
        }
    }
    if (a.n_splits > 1) {
        if (!vec || waves != 2) return (int)hipErrorInvalidValue;
        switch (D) {
            case 32: return launch_twopass_split<T, 32>(mask_kind, a, s);
            case 64: return launch_twopass_split<T, 64>(mask_kind, a, s);
            case 128: return launch_twopass_split<T, 128>(mask_kind, a, s);
            default: return (int)hipErrorInvalidValue;
        }
    }
#define SDPA_TP_DIM(DD)                                                                      \
    case DD:                                                                                 \
        if (!vec) return launch_twopass_mask<T, DD, 2, false, false>(mask_kind, a, s);       \
        if (waves == 4) return launch_twopass_mask<T, DD, 4, true, true>(mask_kind, a, s);   \
        if constexpr (sizeof(T) == 2 || DD < 128) {                                           \
            if (waves == 3) return launch_twopass_mask<T, DD, 3, true, false>(mask_kind, a, s); \
        }                                                                                    \
        if (waves == 2) return launch_twopass_mask<T, DD, 2, true, false>(mask_kind, a, s);  \
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
