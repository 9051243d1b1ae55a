// Backward of the materialised-probability SDPA forward: dq, dk, dv from
// the gradients of both outputs, dout = dL/dO and dprobs = dL/dP.
//
// Math (FlagOS-OP pull request "feat: add sdpa_math operator (Ascend Triton +
// P800 exact-P/A1)": Implementation section, an autograd.Function taking
// both output gradients; "P800 fused backward" update, the softmax Jacobian
// from the probability map and the query-head gradients summed back to the
// key/value heads):
//   P_ij   = exp(S_ij - LSE_i)  (recomputed exactly from the saved LSE, the
//            identity of the page's "P800 exact-P fast path" update)
//   dP_ij  = dout_i . v_j + dprobs_ij
//   D_i    = sum_j P_ij dP_ij
//   dS_ij  = P_ij (dP_ij - D_i)
//   dq_i   = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
//   dv_j   = sum_i P_ij dout_i        (i over every query head of the group)
//
// Two launches, no atomics (every output element has one owner, so results
// are deterministic):
//  * sdpa_bwd_q_kernel: a wave owns 32 query rows; K and V tiles of 32 keys
//    are staged in LDS. Sweep 1 recomputes S^T = K Q^T and dP^T = V dout^T
//    on MFMA (the same keys x queries layout as the forward: each lane holds
//    two runs of 8 consecutive keys of one query row), adds dprobs and folds
//    D_i, which also goes to the workspace; sweep 2 recomputes them, forms
//    dS and accumulates dq^T += K^T dS^T.
//  * sdpa_bwd_kv_kernel: a wave owns 32 keys of one (batch, key/value head)
//    and walks every query head of its group and every query tile (Q, dout,
//    LSE and D staged in LDS): S = Q K^T and dP = dout V^T with queries x
//    keys accumulators (each lane: runs of 8 consecutive queries of one key),
//    then dv^T += dout^T P and dk^T += Q^T dS.
// P and dS enter the 16-bit products as the rounded value plus its rounded
// residual (as in the forward), so the products carry them to twice the
// dtype's precision; scores, row terms and accumulation are float32.

#include <type_traits>

#include "sdpa_device.h"

namespace sdpa {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x2 lds_tr16(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

constexpr int BWQ = 4;  // waves per workgroup of the query-side kernel (128 query rows)
// waves per workgroup of the key-side kernels (64 keys; measured faster than
// 128, whose larger blocks balance the causal triangle worse)
constexpr int BW_KV = 2;

// An LDS tile of rows of D elements: row-major, 16-byte chunks of a row
// permuted in groups of four (chunk c of row r at r * CPR + (c ^ f(r))), so
// that transposing reads of four-row groups stay free of bank conflicts.
template <typename T, int D>
struct Tile {
    static constexpr int SZ = (int)sizeof(T);
    static constexpr int ROWB = D * SZ;
    static constexpr int CPR = ROWB / 16;
    static constexpr int RPB = ROWB >= 256 ? 1 : 256 / ROWB;
    static constexpr int BYTES32 = 32 * ROWB;  // bytes of a 32-row tile
    static_assert(CPR % 4 == 0, "tile rows must hold a multiple of 4 chunks");
    static __device__ __forceinline__ int f(int row) { return 4 * ((row / RPB) & (CPR / 4 - 1)); }
    static __device__ __forceinline__ int pos(int row, int chunk) { return row * CPR + (chunk ^ f(row)); }
};

// Copy rows [row0, row0 + 32) of a slice (row pitch in bytes, rows at or past
// `limit` read as zeros) into a 32-row LDS tile; threads tid, tid + nt, ...
template <typename T, int D>
__device__ __forceinline__ void load_tile32(uint8_t* dst, rsrc_t src, uint32_t pitch, int row0, int limit, int tid,
                                            int nt) {
    using TL = Tile<T, D>;
    for (int i = tid; i < 32 * TL::CPR; i += nt) {
        const int row = i / TL::CPR, c = i - row * TL::CPR;
        const int g = row0 + row;
        const u32x4 x = ld128(src, pred(g < limit, (uint32_t)g * pitch + (uint32_t)(c * 16)));
        *reinterpret_cast<u32x4*>(dst + TL::pos(row, c) * 16) = x;
    }
}

// A 32-row tile's 16-byte chunks held in registers by thread tid of nt
// threads (chunks tid, tid + nt, ...): loaded from global memory one tile
// ahead, written to LDS once the current tile has been consumed, so the
// loads' latency hides behind the current tile's arithmetic.
template <typename T, int D, int NT>
struct Prefetch32 {
    using TL = Tile<T, D>;
    static constexpr int TOTAL = 32 * TL::CPR;
    static constexpr int N = (TOTAL + NT - 1) / NT;
    u32x4 r[N];
    __device__ __forceinline__ void load(rsrc_t src, uint32_t pitch, int row0, int limit, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT;
            if (TOTAL % NT == 0 || idx < TOTAL) {
                const int row = idx / TL::CPR, c = idx - (idx / TL::CPR) * TL::CPR;
                const int g = row0 + row;
                r[i] = ld128(src, pred(g < limit, (uint32_t)g * pitch + (uint32_t)(c * 16)));
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int idx = tid + i * NT;
            if (TOTAL % NT == 0 || idx < TOTAL) {
                const int row = idx / TL::CPR, c = idx - (idx / TL::CPR) * TL::CPR;
                *reinterpret_cast<u32x4*>(dst + TL::pos(row, c) * 16) = r[i];
            }
        }
    }
};

// A operand of an MFMA whose rows are tile rows: lane (m, h) reads tile row
// `row` (the caller passes base + swap23(m)), elements c*KSTEP + h*KH .. +KH.
template <typename T, int D>
__device__ __forceinline__ typename Tr<T>::vec row_operand(const uint8_t* t, int row, int c, int hf) {
    using TL = Tile<T, D>;
    constexpr int KH = Tr<T>::KH;
    const int elem = c * 2 * KH + hf * KH;
    const uint8_t* p = t + TL::pos(row, elem * TL::SZ / 16) * 16 + ((elem * TL::SZ) & 15);
    if constexpr (sizeof(T) == 2) return as_vec<T>(*reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const float*>(p);
}

// One element of a tile (float32 tiles: the transposed A operand).
template <typename T, int D>
__device__ __forceinline__ float tile_elem(const uint8_t* t, int row, int col) {
    using TL = Tile<T, D>;
    return *reinterpret_cast<const float*>(t + TL::pos(row, col * TL::SZ / 16) * 16 + ((col * TL::SZ) & 15));
}

// 16-bit A operand of the transposed tile (A[m][k] = tile[row0 + k][col(m)],
// k over 16 rows, head-dim chunk dd): the gfx950 transposing LDS read; output
// lane i receives column 32 dd + swap23(i % 32), so the product's accumulator
// holds runs of 8 consecutive columns per lane.
template <typename T, int D>
__device__ __forceinline__ typename Tr<T>::vec tr_operand(const uint8_t* t, int row0, int dd, int lane) {
    using TL = Tile<T, D>;
    const int trg = lane >> 4, trs = lane & 15;
    const int sig = ((trs & 1) << 1) | ((trs >> 1) & 1);
    const int trow = 8 * (trg >> 1) + (trs >> 2);
    const int tcol = 16 * (trg & 1) + 4 * sig;
    u32x2 half[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = row0 + trow + 4 * r;
        const int col = 32 * dd + tcol;
        half[r] = lds_tr16(t + TL::pos(row, col * TL::SZ / 16) * 16 + ((col * TL::SZ) & 15));
    }
    return __builtin_bit_cast(typename Tr<T>::vec, u32x4{half[0][0], half[0][1], half[1][0], half[1][1]});
}

// acc^T += tile^T x W for a 32-row block of the tile starting at row0: W is
// the lane's 16 values (two runs of 8 consecutive rows, the accumulator
// layout of a keys x queries or queries x keys product), carried as the
// rounded value plus its rounded residual for 16-bit types.
// `pre` multiplies W before it is split (an exact power of two; the caller
// divides the accumulator by it): fp16 probabilities, at most 1, are lifted
// by 2^12 so that small ones stay out of fp16's subnormal range, where the
// split would carry them only to an absolute 2^-25.
template <typename T, int D>
__device__ __forceinline__ void acc_tr_product(f32x16* acc, const uint8_t* t, int row0, const float* w, int lane,
                                               float pre = 1.0f) {
    using TR = Tr<T>;
    constexpr int ND = D / 32;
    const int n = lane & 31, hf = lane >> 5;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            typename TR::vec a[ND];
#pragma unroll
            for (int dd = 0; dd < ND; ++dd) a[dd] = tr_operand<T, D>(t, row0 + 16 * c2, dd, lane);
            float ws[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ws[e] = w[8 * c2 + e] * pre;
            const typename TR::vec hi = TR::cvt8(ws);
            const typename TR::vec lo = TR::lo8(ws, hi);
#pragma unroll
            for (int dd = 0; dd < ND; ++dd) acc[dd] = TR::mfma(a[dd], hi, acc[dd]);
#pragma unroll
            for (int dd = 0; dd < ND; ++dd) acc[dd] = TR::mfma(a[dd], lo, acc[dd]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = row0 + kk(hf, r);
#pragma unroll
            for (int dd = 0; dd < ND; ++dd)
                acc[dd] = TR::mfma(tile_elem<T, D>(t, row, 32 * dd + swap23(n)), w[r], acc[dd]);
        }
    }
}

// Store a lane's D-column accumulator (runs of 8 consecutive columns) to
// row `row_off` of a descriptor, times `mul`, rounded to T.
template <typename T, int D>
__device__ __forceinline__ void store_acc_row(rsrc_t r, uint32_t row_off, bool ok, const f32x16* acc, float mul, int hf) {
#pragma unroll
    for (int dd = 0; dd < D / 32; ++dd) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = acc[dd][e] * mul;
        store8<T, true>(r, row_off, ok, 32 * dd + 8 * hf, D, x);
        store8<T, true>(r, row_off, ok, 32 * dd + 16 + 8 * hf, D, x + 8);
    }
}

// B operand held by a lane for row n of a slice: elements c*KSTEP + h*KH ..
template <typename T, int D>
__device__ __forceinline__ void load_frags(typename Tr<T>::vec* f, rsrc_t r, uint32_t row_off, bool ok, int hf) {
    constexpr int KH = Tr<T>::KH;
#pragma unroll
    for (int c = 0; c < D / (2 * KH); ++c) {
        const uint32_t off = pred(ok, row_off + (uint32_t)((c * 2 * KH + hf * KH) * (int)sizeof(T)));
        if constexpr (sizeof(T) == 2) f[c] = as_vec<T>(ld128(r, off));
        else f[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
}

// dprobs of lane (n, h) in a keys x queries block: row `row_off`, keys
// jb + kk(h, r) (past Skv: 0).
template <typename T>
__device__ __forceinline__ void load_dprobs16(const BwdArgs& a, rsrc_t r, uint32_t row_off, bool row_ok, int jb, int hf,
                                              float* out) {
    constexpr int SZ = (int)sizeof(T);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int j = jb + 16 * c + 8 * hf;
        if (a.dp_vec) {
            const uint32_t off = pred(row_ok && j < a.f.Skv, row_off + (uint32_t)(j * SZ));
            if constexpr (SZ == 2) {
                const u32x4 w = ld128(r, off);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[8 * c + e] = Tr<T>::to_f((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            } else {
                const u32x4 w0 = ld128(r, off);
                const u32x4 w1 = ld128(r, off == OOB ? OOB : off + 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t b0 = w0[e], b1 = w1[e];
                    out[8 * c + e] = __builtin_bit_cast(float, b0);
                    out[8 * c + 4 + e] = __builtin_bit_cast(float, b1);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = pred(row_ok && j + e < a.f.Skv, row_off + (uint32_t)((j + e) * SZ));
                if constexpr (SZ == 2) out[8 * c + e] = Tr<T>::to_f(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
                else out[8 * c + e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
            }
        }
    }
}

// One mask element (base-2 additive term: a bool mask gives 0 where it keeps
// the key, -inf where it removes it).
template <typename T, int MASK>
__device__ __forceinline__ float mask_elem(const FwdArgs& f, rsrc_t mr, int qi, int j) {
    constexpr int ME = MASK == MASK_BOOL ? 1 : (int)sizeof(T);
    const uint32_t off = (uint32_t)(((int64_t)qi * f.m_s[2] + (int64_t)j * f.m_s[3]) * ME);
    if constexpr (MASK == MASK_BOOL) {
        return __builtin_amdgcn_raw_buffer_load_b8(mr, off, 0, 0) ? 0.0f : -INFINITY;
    } else if constexpr (sizeof(T) == 2) {
        return Tr<T>::to_f(__builtin_amdgcn_raw_buffer_load_b16(mr, off, 0, 0)) * LOG2E;
    } else {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mr, off, 0, 0)) * LOG2E;
    }
}

// ====================================================================== dq

template <typename T, int D, int MASK, bool HAS_DP>
__global__ __launch_bounds__(BWQ * 64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && MASK != MASK_NONE ? 2 : 1)))
void sdpa_bwd_q_kernel(const BwdArgs a) {
    using TR = Tr<T>;
    using vec = typename TR::vec;
    using TL = Tile<T, D>;
    constexpr int SZ = (int)sizeof(T);
    constexpr int KH = TR::KH;
    constexpr int NKS = D / (2 * KH);
    constexpr int ND = D / 32;
    constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;
    const FwdArgs& f = a.f;

    // 16-bit, D = 128: each wave's q and dout rows live in LDS (read as B
    // operands per tile) instead of 64 registers, which lets two waves share
    // a SIMD (2k causal bf16: 816 -> 700 us). With a mask the per-lane mask
    // and dprobs loads need the occupancy request above as well (the
    // compiler otherwise spends the freed registers on them): GQA key
    // padding 2077 -> 1845 us. Smaller head dims already run two or more per
    // SIMD (1k D = 64: 183 -> 193 us with the rows in LDS).
    constexpr bool DO_LDS = sizeof(T) == 2 && D == 128;
    __shared__ __attribute__((aligned(16))) uint8_t smem[(2 + (DO_LDS ? 2 * BWQ : 0)) * TL::BYTES32];
    uint8_t* kt = smem;
    uint8_t* vt = smem + TL::BYTES32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hf = lane >> 5;
    // causal: query-block major, the last (heaviest) blocks of every head
    // first (2k causal bf16: 676 -> 623 us); otherwise head-major
    const int nqb = (f.Sq + 32 * BWQ - 1) / (32 * BWQ);
    const int nbh = f.B * f.Hq;
    const int bh = f.causal ? (int)blockIdx.x % nbh : (int)blockIdx.x / nqb;
    const int qblk = f.causal ? nqb - 1 - (int)blockIdx.x / nbh : (int)blockIdx.x - bh * nqb;
    const int b = bh / f.Hq, h = bh - (bh / f.Hq) * f.Hq;
    const int hk = h / f.group;
    const int q0 = qblk * 32 * BWQ;
    const int qw = q0 + 32 * wave;
    const int qi = qw + n;
    const bool row_ok = qi < f.Sq;
    const int kend = f.causal ? min(f.Skv, max(0, q0 + 32 * BWQ + f.coff)) : f.Skv;
    const int ntiles = (kend + 31) / 32;

    const rsrc_t qr = make_rsrc(static_cast<const T*>(f.q) + b * f.q_s[0] + h * f.q_s[1], f.q_ext);
    const rsrc_t kr = make_rsrc(static_cast<const T*>(f.k) + b * f.k_s[0] + hk * f.k_s[1], f.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(f.v) + b * f.v_s[0] + hk * f.v_s[1], f.v_ext);
    const rsrc_t dor = make_rsrc(static_cast<const T*>(a.dout) + b * a.do_s[0] + h * a.do_s[1], a.do_ext);
    const rsrc_t dqr = make_rsrc(static_cast<T*>(a.dq) + b * a.dq_s[0] + h * a.dq_s[1], a.dq_ext);
    rsrc_t dpr = qr, mr = qr;
    if constexpr (HAS_DP) dpr = make_rsrc(static_cast<const T*>(a.dprobs) + b * a.dp_s[0] + h * a.dp_s[1], a.dp_ext);
    if constexpr (MASK != MASK_NONE)
        mr = make_rsrc(static_cast<const uint8_t*>(f.mask) + (b * f.m_s[0] + h * f.m_s[1]) * ME, f.m_ext);

    vec qf[DO_LDS ? 1 : NKS], df[DO_LDS ? 1 : NKS];
    uint8_t* qtw = smem + (2 + wave) * TL::BYTES32;        // this wave's q rows (16-bit)
    uint8_t* dtw = smem + (2 + BWQ + wave) * TL::BYTES32;  // and dout rows
    if constexpr (DO_LDS) {
        // the lane's fragments, written where row_operand(.., n, c, hf) reads them
        vec fr[NKS];
        load_frags<T, D>(fr, qr, (uint32_t)(row_ok ? qi : 0) * (uint32_t)(f.q_s[2] * SZ), row_ok, hf);
#pragma unroll
        for (int c = 0; c < NKS; ++c)
            *reinterpret_cast<u32x4*>(qtw + TL::pos(n, 2 * c + hf) * 16) = __builtin_bit_cast(u32x4, fr[c]);
        load_frags<T, D>(fr, dor, (uint32_t)(row_ok ? qi : 0) * (uint32_t)(a.do_s[2] * SZ), row_ok, hf);
#pragma unroll
        for (int c = 0; c < NKS; ++c)
            *reinterpret_cast<u32x4*>(dtw + TL::pos(n, 2 * c + hf) * 16) = __builtin_bit_cast(u32x4, fr[c]);
    } else {
        load_frags<T, D>(qf, qr, (uint32_t)(row_ok ? qi : 0) * (uint32_t)(f.q_s[2] * SZ), row_ok, hf);
        load_frags<T, D>(df, dor, (uint32_t)(row_ok ? qi : 0) * (uint32_t)(a.do_s[2] * SZ), row_ok, hf);
    }
    float lse2 = INFINITY;  // dead or absent rows: every probability exp2(-inf) = 0
    if (row_ok) {
        const float l = f.lse[b * f.l_s[0] + h * f.l_s[1] + (int64_t)qi * f.l_s[2]];
        lse2 = l == -INFINITY ? INFINITY : l * LOG2E;
    }
    const uint32_t dp_row = (uint32_t)(row_ok ? qi : 0) * (uint32_t)(a.dp_s[2] * SZ);
    const uint32_t m_row = (uint32_t)((int64_t)(row_ok ? qi : 0) * f.m_s[2] * ME);
    const uint32_t krow = (uint32_t)(f.k_s[2] * SZ), vrow = (uint32_t)(f.v_s[2] * SZ);

    Prefetch32<T, D, BWQ * 64> kp, vp;
    auto prefetch = [&](int t) __attribute__((always_inline)) {
        kp.load(kr, krow, t * 32, f.Skv, tid);
        vp.load(vr, vrow, t * 32, f.Skv, tid);
    };
    // the per-lane loads of tile t (mask terms, dprobs): issued before the
    // next tile's prefetch, so waiting for them does not wait for it
    auto lane_loads = [&](int t, float* mv, float* dpv) __attribute__((always_inline)) {
        if constexpr (MASK != MASK_NONE) {
            if (f.mask_vec) load_mask16<T, MASK, true>(f, mr, m_row, t * 32, hf, mv);  // one load per 8 keys
            else load_mask16<T, MASK, false>(f, mr, m_row, t * 32, hf, mv);
        }
        if constexpr (HAS_DP) load_dprobs16<T>(a, dpr, dp_row, row_ok, t * 32, hf, dpv);
    };
    // probabilities and gradient-at-P of this lane's 16 (query, key) pairs of
    // the staged 32-key tile t; removed keys give P = 0
    auto block = [&](int t, const float* mv, const float* dpv, float* p, float* dp) __attribute__((always_inline)) {
        const int jb = t * 32;
        f32x16 s = {}, g = {};
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            if constexpr (DO_LDS) s = TR::mfma(row_operand<T, D>(kt, swap23(n), c, hf), row_operand<T, D>(qtw, n, c, hf), s);
            else s = TR::mfma(row_operand<T, D>(kt, swap23(n), c, hf), qf[c], s);
        }
#pragma unroll
        for (int c = 0; c < NKS; ++c) {
            if constexpr (DO_LDS) g = TR::mfma(row_operand<T, D>(vt, swap23(n), c, hf), row_operand<T, D>(dtw, n, c, hf), g);
            else g = TR::mfma(row_operand<T, D>(vt, swap23(n), c, hf), df[c], g);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = jb + kk(hf, r);
            float x = MASK != MASK_NONE ? __builtin_fmaf(s[r], f.scale_log2, mv[r]) : s[r] * f.scale_log2;
            if (j >= f.Skv || (f.causal && j > qi + f.coff)) x = -INFINITY;
            p[r] = fast_exp2(x - lse2);
            dp[r] = HAS_DP ? g[r] + dpv[r] : g[r];
        }
    };
    // one sweep over the key tiles: the first tile staged, then per tile the
    // lane loads, the next tile's prefetch, the arithmetic, and the handover
    auto sweep = [&](auto&& body) __attribute__((always_inline)) {
        if (ntiles > 0) {
            prefetch(0);
            kp.store(kt, tid);
            vp.store(vt, tid);
        }
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            float mv[16], dpv[16];
            lane_loads(t, mv, dpv);
            if (t + 1 < ntiles) prefetch(t + 1);
            // a tile whose mask removes every key of this wave's rows adds
            // nothing (P = 0 there): its products are skipped
            bool live = true;
            if constexpr (MASK != MASK_NONE) {
                bool any = false;
#pragma unroll
                for (int r = 0; r < 16; ++r) any |= mv[r] != -INFINITY;
                live = __builtin_amdgcn_ballot_w64(any && row_ok) != 0;
            }
            if (live) {
                float p[16], dp[16];
                block(t, mv, dpv, p, dp);
                body(p, dp);
            }
            __syncthreads();  // tile t consumed
            if (t + 1 < ntiles) {
                kp.store(kt, tid);
                vp.store(vt, tid);
            }
            __syncthreads();
        }
    };

    // ---------------- sweep 1: D_i = sum_j P_ij dP_ij
    float dsum = 0.0f;
    sweep([&](const float* p, const float* dp) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dsum = __builtin_fmaf(p[r], dp[r], dsum);
    });
    dsum += __shfl_xor(dsum, 32);
    if (row_ok && hf == 0) a.dsum[((int64_t)b * f.Hq + h) * f.Sq + qi] = dsum;

    // ---------------- sweep 2: dS = P (dP - D); dq^T += K^T dS^T
    f32x16 acc[ND];
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) acc[dd] = f32x16{};
    sweep([&](const float* p, const float* dp) __attribute__((always_inline)) {
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dp[r] - dsum);
        acc_tr_product<T, D>(acc, kt, 0, ds, lane);
    });
    store_acc_row<T, D>(dqr, (uint32_t)(row_ok ? qi : 0) * (uint32_t)(a.dq_s[2] * SZ), row_ok, acc, a.scale, hf);
}

// ====================================================================== dk, dv

// WHICH: KV_DV accumulates dv only (S, P), KV_DK dk only (S, P, dP, dS),
// KV_BOTH both. The two single-gradient launches hold half the accumulators,
// so twice the waves fit per SIMD: faster despite recomputing S once the grid
// is large enough to fill the chip twice over; below that one launch wins.
constexpr int KV_DV = 1, KV_DK = 2, KV_BOTH = 3;

template <typename T, int D, int MASK, bool HAS_DP, int WHICH>
__global__ __launch_bounds__(BW_KV * 64) __attribute__((amdgpu_waves_per_eu(WHICH != KV_BOTH && sizeof(T) == 2 && !(D == 128 && MASK != MASK_NONE && HAS_DP) ? 2 : 1)))
void sdpa_bwd_kv_kernel(const BwdArgs a) {
    constexpr int BW = BW_KV;
    constexpr bool DO_DV = (WHICH & KV_DV) != 0;
    constexpr bool NEED_DP = (WHICH & KV_DK) != 0;  // dP, dprobs and D: dk only
    using TR = Tr<T>;
    using TL = Tile<T, D>;
    constexpr int SZ = (int)sizeof(T);
    constexpr int KH = TR::KH;
    constexpr int NKS = D / (2 * KH);
    constexpr int ND = D / 32;
    constexpr int ME = MASK == MASK_BOOL ? 1 : SZ;
    constexpr float P_LIFT = std::is_same<T, _Float16>::value ? 4096.0f : 1.0f;
    const FwdArgs& f = a.f;

    // Q and dout tiles of the current 32 query rows, their log2-domain LSE and
    // D, then per wave its 32 key rows of K and V and its dprobs tile
    // (the dv pass reads neither V nor dprobs)
    constexpr int DPB = HAS_DP && NEED_DP ? 32 * 32 * SZ : 0;  // dprobs tile: 32 queries x 32 keys
    constexpr int WAVEB = (NEED_DP ? 2 : 1) * TL::BYTES32 + DPB;
    // mask tile of a step (aligned contiguous masks): its 32 query rows x the
    // workgroup's 32 BW keys, staged with Q and dout by whole-row loads and
    // read back by column (each lane's key)
    constexpr int MROW = 32 * BW * ME;
    constexpr int MTB = MASK != MASK_NONE ? 32 * MROW : 0;
    constexpr int MCH = MTB / 16 / (BW * 64);  // 16-byte chunks per thread
    static_assert(MTB % (16 * BW * 64) == 0, "mask tile chunks must split evenly over the threads");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::BYTES32 + 2 * 32 * 4 + BW * WAVEB + MTB];
    uint8_t* qt = smem;
    uint8_t* dot = smem + TL::BYTES32;
    float* lse_s = reinterpret_cast<float*>(smem + 2 * TL::BYTES32);
    float* dsum_s = lse_s + 32;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hf = lane >> 5;
    uint8_t* kw = smem + 2 * TL::BYTES32 + 2 * 32 * 4 + wave * WAVEB;
    uint8_t* mtile = smem + 2 * TL::BYTES32 + 2 * 32 * 4 + BW * WAVEB;
    uint8_t* vw = kw + TL::BYTES32;
    uint8_t* dpw = vw + TL::BYTES32;

    const int nkb = (f.Skv + 32 * BW - 1) / (32 * BW);
    // key block major: the early key blocks (the most query tiles under a
    // causal mask) of every head go first; with query ranges the ranges of
    // a key block are consecutive
    const int ns = WHICH == KV_BOTH ? a.kv_splits : 1;
    const int sidx = ns > 1 ? (int)blockIdx.x % ns : 0;
    const int lin = ns > 1 ? (int)blockIdx.x / ns : (int)blockIdx.x;
    const int nbk = f.B * f.Hkv;
    const int kblk = lin / nbk;
    const int bk = lin - kblk * nbk;
    const int b = bk / f.Hkv, hk = bk - (bk / f.Hkv) * f.Hkv;
    const int k0 = kblk * 32 * BW;
    const int kw0 = k0 + 32 * wave;
    const int kj = kw0 + n;  // this lane's key
    const bool key_ok = kj < f.Skv;

    const rsrc_t kr = make_rsrc(static_cast<const T*>(f.k) + b * f.k_s[0] + hk * f.k_s[1], f.k_ext);
    const rsrc_t vr = make_rsrc(static_cast<const T*>(f.v) + b * f.v_s[0] + hk * f.v_s[1], f.v_ext);
    const rsrc_t dkr = make_rsrc(static_cast<T*>(a.dk) + b * a.dk_s[0] + hk * a.dk_s[1], a.dk_ext);
    const rsrc_t dvr = make_rsrc(static_cast<T*>(a.dv) + b * a.dv_s[0] + hk * a.dv_s[1], a.dv_ext);

    // this wave's key rows (B operands of both products)
    load_tile32<T, D>(kw, kr, (uint32_t)(f.k_s[2] * SZ), kw0, f.Skv, lane, 64);
    if constexpr (NEED_DP) load_tile32<T, D>(vw, vr, (uint32_t)(f.v_s[2] * SZ), kw0, f.Skv, lane, 64);

    // dk^T, dv^T of this lane's key (what this launch accumulates)
    f32x16 dk[NEED_DP ? ND : 1], dv[DO_DV ? ND : 1];
#pragma unroll
    for (int dd = 0; dd < ND; ++dd) {
        if constexpr (NEED_DP) dk[dd] = f32x16{};
        if constexpr (DO_DV) dv[dd] = f32x16{};
    }
    // causal: query i sees key j iff j <= i + coff, so queries below
    // k0 - coff see none of this workgroup's keys
    const int qstart = f.causal ? max(0, k0 - f.coff) / 32 * 32 : 0;
    const int nqt = f.Sq > qstart ? (f.Sq - qstart + 31) / 32 : 0;  // query tiles per head
    const int nit_all = f.group * nqt;                               // (head of the group, query tile) steps
    // this workgroup's steps [it_lo, nit) (all of them without query ranges)
    const int per = (nit_all + ns - 1) / ns;
    const int it_lo = min(nit_all, sidx * per);
    const int nit = min(nit_all, it_lo + per);

    // the next step's tiles, held in registers until the current one is consumed
    Prefetch32<T, D, BW * 64> qp, dop;
    float lse_n = INFINITY, dsum_n = 0.0f;  // thread tid < 32: row i0 + tid of the next step
    constexpr int DPC = 32 * 32 * SZ / 16 / 64;  // 16-byte chunks of a dprobs tile per lane
    u32x4 dpn[DPC];
    [[maybe_unused]] u32x4 mpn[MCH > 0 ? MCH : 1];
    auto step_coords = [&](int it, int& h, int& i0) __attribute__((always_inline)) {
        const int hh = it / nqt;
        h = hk * f.group + hh;
        i0 = qstart + (it - hh * nqt) * 32;
    };
    auto prefetch = [&](int it) __attribute__((always_inline)) {
        int h, i0;
        step_coords(it, h, i0);
        const rsrc_t qr = make_rsrc(static_cast<const T*>(f.q) + b * f.q_s[0] + h * f.q_s[1], f.q_ext);
        const rsrc_t dor = make_rsrc(static_cast<const T*>(a.dout) + b * a.do_s[0] + h * a.do_s[1], a.do_ext);
        qp.load(qr, (uint32_t)(f.q_s[2] * SZ), i0, f.Sq, tid);
        dop.load(dor, (uint32_t)(a.do_s[2] * SZ), i0, f.Sq, tid);
        if constexpr (MASK != MASK_NONE) {
            if (f.mask_vec) {
                const rsrc_t mrh = make_rsrc(static_cast<const uint8_t*>(f.mask) + (b * f.m_s[0] + h * f.m_s[1]) * ME, f.m_ext);
#pragma unroll
                for (int u = 0; u < MCH; ++u) {
                    const int idx = tid + u * BW * 64;
                    const int rr = idx / (MROW / 16), cc = idx - (idx / (MROW / 16)) * (MROW / 16);
                    const int i = i0 + rr, j = k0 + cc * (16 / ME);
                    mpn[u] = ld128(mrh, pred(i < f.Sq && j < f.Skv, (uint32_t)(((int64_t)i * f.m_s[2] + j) * ME)));
                }
            }
        }
        if (tid < 32) {
            const int i = i0 + tid;
            const float l = i < f.Sq ? f.lse[b * f.l_s[0] + h * f.l_s[1] + (int64_t)i * f.l_s[2]] : -INFINITY;
            lse_n = l == -INFINITY ? INFINITY : l * LOG2E;
            if constexpr (NEED_DP) dsum_n = i < f.Sq ? a.dsum[((int64_t)b * f.Hq + h) * f.Sq + i] : 0.0f;
        }
        if constexpr (HAS_DP && NEED_DP) {
            // rows i0 .. i0+31, this wave's 32 keys: 16-byte chunks when the
            // rows allow it, else element by element (into the same chunks)
            const rsrc_t dpr = make_rsrc(static_cast<const T*>(a.dprobs) + b * a.dp_s[0] + h * a.dp_s[1], a.dp_ext);
            constexpr int CPRD = 32 * SZ / 16;  // chunks per tile row
#pragma unroll
            for (int u = 0; u < DPC; ++u) {
                const int idx = lane + 64 * u;
                const int rr = idx / CPRD, cc = idx - (idx / CPRD) * CPRD;
                const int i = i0 + rr, j = kw0 + cc * (16 / SZ);
                const uint32_t row_off = (uint32_t)i * (uint32_t)(a.dp_s[2] * SZ);
                if (a.dp_vec) {
                    dpn[u] = ld128(dpr, pred(i < f.Sq && j < f.Skv, row_off + (uint32_t)(j * SZ)));
                } else {
                    uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 16 / SZ; ++e) {
                        const uint32_t off = pred(i < f.Sq && j + e < f.Skv, row_off + (uint32_t)((j + e) * SZ));
                        if constexpr (SZ == 2)
                            wv[e >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(dpr, off, 0, 0) << (16 * (e & 1));
                        else
                            wv[e] = __builtin_amdgcn_raw_buffer_load_b32(dpr, off, 0, 0);
                    }
                    dpn[u] = u32x4{wv[0], wv[1], wv[2], wv[3]};
                }
            }
        }
    };
    auto put = [&]() __attribute__((always_inline)) {
        qp.store(qt, tid);
        dop.store(dot, tid);
        if constexpr (MASK != MASK_NONE) {
            if (f.mask_vec) {
#pragma unroll
                for (int u = 0; u < MCH; ++u) reinterpret_cast<u32x4*>(mtile)[tid + u * BW * 64] = mpn[u];
            }
        }
        if (tid < 32) {
            lse_s[tid] = lse_n;
            dsum_s[tid] = dsum_n;
        }
        if constexpr (HAS_DP && NEED_DP) {
#pragma unroll
            for (int u = 0; u < DPC; ++u) reinterpret_cast<u32x4*>(dpw)[lane + 64 * u] = dpn[u];
        }
    };

    if (nit > it_lo) {
        prefetch(it_lo);
        put();
    }
    __syncthreads();  // (also orders this wave's K and V rows before their first reads)
    for (int it = it_lo; it < nit; ++it) {
        int h, i0;
        step_coords(it, h, i0);
        // this step's mask terms (per lane: its key, 16 queries), before the prefetch
        float mv[16];
        if constexpr (MASK != MASK_NONE) {
            if (f.mask_vec) {  // from the staged tile: row kk(hf, r), this lane's key
                const uint8_t* mc = mtile + (kj - k0) * ME;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = i0 + kk(hf, r);
                    const uint8_t* e = mc + kk(hf, r) * MROW;
                    float x;
                    if constexpr (MASK == MASK_BOOL) x = *e ? 0.0f : -INFINITY;
                    else if constexpr (SZ == 2) x = Tr<T>::to_f(*reinterpret_cast<const uint16_t*>(e)) * LOG2E;
                    else x = *reinterpret_cast<const float*>(e) * LOG2E;
                    mv[r] = (i < f.Sq && key_ok) ? x : 0.0f;
                }
            } else {
                const rsrc_t mr = make_rsrc(static_cast<const uint8_t*>(f.mask) + (b * f.m_s[0] + h * f.m_s[1]) * ME, f.m_ext);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = i0 + kk(hf, r);
                    mv[r] = (i < f.Sq && key_ok) ? mask_elem<T, MASK>(f, mr, i, kj) : 0.0f;
                }
            }
        }
        if (it + 1 < nit) prefetch(it + 1);

        // S = Q K^T and dP = dout V^T: lane (n, h) holds queries
        // i0 + kk(h, r) of key kj
        f32x16 sacc = {}, g = {};
#pragma unroll
        for (int c = 0; c < NKS; ++c)
            sacc = TR::mfma(row_operand<T, D>(qt, swap23(n), c, hf), row_operand<T, D>(kw, n, c, hf), sacc);
        if constexpr (NEED_DP) {
#pragma unroll
            for (int c = 0; c < NKS; ++c)
                g = TR::mfma(row_operand<T, D>(dot, swap23(n), c, hf), row_operand<T, D>(vw, n, c, hf), g);
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ql = kk(hf, r);
            const int i = i0 + ql;
            float x = MASK != MASK_NONE ? __builtin_fmaf(sacc[r], f.scale_log2, mv[r]) : sacc[r] * f.scale_log2;
            if (!key_ok || (f.causal && kj > i + f.coff)) x = -INFINITY;
            p[r] = fast_exp2(x - lse_s[ql]);
            if constexpr (NEED_DP) {
                float dp = g[r];
                if constexpr (HAS_DP) {
                    if constexpr (SZ == 2) dp += Tr<T>::to_f(reinterpret_cast<const uint16_t*>(dpw)[ql * 32 + n]);
                    else dp += reinterpret_cast<const float*>(dpw)[ql * 32 + n];
                }
                ds[r] = p[r] * (dp - dsum_s[ql]);
            }
        }
        if constexpr (DO_DV) acc_tr_product<T, D>(dv, dot, 0, p, lane, P_LIFT);
        if constexpr (NEED_DP) acc_tr_product<T, D>(dk, qt, 0, ds, lane);
        __syncthreads();  // step consumed
        if (it + 1 < nit) put();
        __syncthreads();
    }
    if constexpr (WHICH == KV_BOTH) {
        if (ns > 1) {  // float32 partials of this query range, unscaled
            const int64_t plane = (int64_t)nbk * f.Skv * D;
            float* pk = a.ws_kv + ((int64_t)sidx * nbk + bk) * f.Skv * D + (int64_t)(key_ok ? kj : 0) * D;
            float* pv = pk + (int64_t)ns * plane;
            if (key_ok) {
#pragma unroll
                for (int dd = 0; dd < ND; ++dd) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int c0 = 32 * dd + 16 * h2 + 8 * hf;
#pragma unroll
                        for (int q4 = 0; q4 < 2; ++q4) {
                            const int e = 8 * h2 + 4 * q4;
                            *reinterpret_cast<f32x4*>(pk + c0 + 4 * q4) =
                                f32x4{dk[dd][e], dk[dd][e + 1], dk[dd][e + 2], dk[dd][e + 3]};
                            *reinterpret_cast<f32x4*>(pv + c0 + 4 * q4) =
                                f32x4{dv[dd][e], dv[dd][e + 1], dv[dd][e + 2], dv[dd][e + 3]};
                        }
                    }
                }
            }
            return;
        }
    }
    const uint32_t krow_off = (uint32_t)(key_ok ? kj : 0);
    if constexpr (NEED_DP) store_acc_row<T, D>(dkr, krow_off * (uint32_t)(a.dk_s[2] * SZ), key_ok, dk, a.scale, hf);
    if constexpr (DO_DV) store_acc_row<T, D>(dvr, krow_off * (uint32_t)(a.dv_s[2] * SZ), key_ok, dv, 1.0f / P_LIFT, hf);
}

// dk and dv of a key-side launch over query ranges: each row's float32
// partials summed in range order, then scaled (dk: the score scale; dv: the
// fp16 probability lift undone) and rounded once. One thread per 8
// consecutive columns of a (batch, KV head, key) row.
template <typename T>
__global__ __launch_bounds__(256) void sdpa_bwd_kv_reduce_kernel(const BwdArgs a, int D) {
    const FwdArgs& f = a.f;
    constexpr float P_LIFT = std::is_same<T, _Float16>::value ? 4096.0f : 1.0f;
    const int nbk = f.B * f.Hkv;
    const int64_t rows = (int64_t)nbk * f.Skv;
    const int cpr = D / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * cpr) return;
    const int64_t row = i / cpr;
    const int c = (int)(i - row * cpr) * 8;
    const int bk = (int)(row / f.Skv), key = (int)(row - (int64_t)bk * f.Skv);
    const int b = bk / f.Hkv, hk = bk - (bk / f.Hkv) * f.Hkv;
    const int64_t plane = rows * D;
    float sk[8] = {0, 0, 0, 0, 0, 0, 0, 0}, sv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s2 = 0; s2 < a.kv_splits; ++s2) {
        const float* pk = a.ws_kv + (int64_t)s2 * plane + row * D + c;
        const float* pv = pk + (int64_t)a.kv_splits * plane;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 uk = *reinterpret_cast<const f32x4*>(pk + 4 * h);
            const f32x4 uv = *reinterpret_cast<const f32x4*>(pv + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk[4 * h + e] += uk[e];
                sv[4 * h + e] += uv[e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sk[e] *= a.scale;
        sv[e] *= 1.0f / P_LIFT;
    }
    T* dk = static_cast<T*>(a.dk) + b * a.dk_s[0] + hk * a.dk_s[1] + (int64_t)key * a.dk_s[2] + c;
    T* dv = static_cast<T*>(a.dv) + b * a.dv_s[0] + hk * a.dv_s[1] + (int64_t)key * a.dv_s[2] + c;
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(dk) = __builtin_bit_cast(u32x4, Tr<T>::cvt8(sk));
        *reinterpret_cast<u32x4*>(dv) = __builtin_bit_cast(u32x4, Tr<T>::cvt8(sv));
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<f32x4*>(dk + 4 * h) = f32x4{sk[4 * h], sk[4 * h + 1], sk[4 * h + 2], sk[4 * h + 3]};
            *reinterpret_cast<f32x4*>(dv + 4 * h) = f32x4{sv[4 * h], sv[4 * h + 1], sv[4 * h + 2], sv[4 * h + 3]};
        }
    }
}

// Key-side launches: split into a dk and a dv pass once each pass alone has
// at least two waves per SIMD of the chip (256 CUs x 4 SIMDs), one combined
// pass below that.
constexpr int64_t KV_SPLIT_MIN_WAVES = 2 * 256 * 4;

template <typename T, int D, int MASK, bool HAS_DP>
void launch_bwd_kv(const BwdArgs& a, int64_t nk, hipStream_t s) {
    if (nk <= 0) return;
    if (nk * BW_KV >= KV_SPLIT_MIN_WAVES) {
        hipLaunchKernelGGL((sdpa_bwd_kv_kernel<T, D, MASK, HAS_DP, KV_DK>), dim3((unsigned)nk), dim3(BW_KV * 64), 0, s, a);
        hipLaunchKernelGGL((sdpa_bwd_kv_kernel<T, D, MASK, HAS_DP, KV_DV>), dim3((unsigned)nk), dim3(BW_KV * 64), 0, s, a);
    } else {
        const int ns = a.kv_splits > 1 ? a.kv_splits : 1;
        hipLaunchKernelGGL((sdpa_bwd_kv_kernel<T, D, MASK, HAS_DP, KV_BOTH>), dim3((unsigned)(nk * ns)),
                           dim3(BW_KV * 64), 0, s, a);
        if (ns > 1) {
            const int64_t n = (int64_t)a.f.B * a.f.Hkv * a.f.Skv * (D / 8);
            hipLaunchKernelGGL(sdpa_bwd_kv_reduce_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, D);
        }
    }
}

template <typename T, int D, int MASK>
int launch_bwd_t(const BwdArgs& a, hipStream_t s) {
    const int64_t nq = (int64_t)a.f.B * a.f.Hq * ((a.f.Sq + 32 * BWQ - 1) / (32 * BWQ));
    const int64_t nk = (int64_t)a.f.B * a.f.Hkv * ((a.f.Skv + 32 * BW_KV - 1) / (32 * BW_KV));
    if (a.dprobs) {
        if (nq > 0) hipLaunchKernelGGL((sdpa_bwd_q_kernel<T, D, MASK, true>), dim3((unsigned)nq), dim3(BWQ * 64), 0, s, a);
        launch_bwd_kv<T, D, MASK, true>(a, nk, s);
    } else {
        if (nq > 0) hipLaunchKernelGGL((sdpa_bwd_q_kernel<T, D, MASK, false>), dim3((unsigned)nq), dim3(BWQ * 64), 0, s, a);
        launch_bwd_kv<T, D, MASK, false>(a, nk, s);
    }
    return (int)hipGetLastError();
}

template <typename T, int D>
int launch_bwd_d(int mask_kind, const BwdArgs& a, hipStream_t s) {
    switch (mask_kind) {
        case MASK_NONE: return launch_bwd_t<T, D, MASK_NONE>(a, s);
        case MASK_BOOL: return launch_bwd_t<T, D, MASK_BOOL>(a, s);
        case MASK_ADD: return launch_bwd_t<T, D, MASK_ADD>(a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

template <typename T>
int launch_bwd_dt(int D, int mask_kind, const BwdArgs& a, hipStream_t s) {
    switch (D) {
        case 32: return launch_bwd_d<T, 32>(mask_kind, a, s);
        case 64: return launch_bwd_d<T, 64>(mask_kind, a, s);
        case 128: return launch_bwd_d<T, 128>(mask_kind, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_backward(int dtype, int D, int mask_kind, const BwdArgs& a, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (dtype) {
        case DT_F32: return launch_bwd_dt<float>(D, mask_kind, a, s);
        case DT_F16: return launch_bwd_dt<_Float16>(D, mask_kind, a, s);
        case DT_BF16: return launch_bwd_dt<__bf16>(D, mask_kind, a, s);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace sdpa
