// Device-side building blocks shared by the gfx950 kernels.
//
// Layout trick used by every kernel: a wave computes S^T = K Q^T for 32 keys
// x 32 queries with v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2_f32
// for float32). Lane l owns query column n = l % 32 and half h = l / 32.
// Loading MFMA row m of the K operand from key swap23(m) (bits 2 and 3 of m
// exchanged) makes accumulator register r of lane (n, h) hold key
//     kk(h, r) = r < 8 ? 8h + r : 16 + 8h + (r - 8)
// so each lane ends up with two runs of 8 consecutive keys of ONE query row:
//   * row statistics are lane-local plus one exchange with lane l ^ 32;
//   * the rounded probabilities are already the B operand of the next MFMA,
//     O^T += V^T P^T, with no LDS round trip (slot j of half h = key 16c+8h+j);
//   * every lane stores P as 16-byte row chunks.
// The same permutation on the V^T rows makes the O^T accumulator hold runs
// of 8 consecutive head-dim columns per lane.
//
// Global memory is reached through buffer descriptors covering one
// (batch, head) slice. A lane whose element is out of range is given an
// offset past the descriptor's end: the hardware then drops the store or
// returns zero for the load, so ragged edges need no branches and the
// compiler's memory-counter waits stay exact (loads issued before the
// probability stores of a tile are waited for without waiting on those
// stores).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_internal.h"

namespace sdpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int BN = TILE_N;                  // keys per tile (two 32-key MFMA blocks)
constexpr uint32_t OOB = 0x80000000u;       // offset past every descriptor's end
constexpr int32_t RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data, gfx9-family

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ constexpr int kk(int h, int r) { return r < 8 ? 8 * h + r : 16 + 8 * h + (r - 8); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, RSRC_WORD3);
}
__device__ __forceinline__ uint32_t pred(bool ok, uint32_t off) { return ok ? off : OOB; }

__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }
// A 16-byte store reads its data registers after issue; the following
// instruction must not rewrite them. The s_nop below (two wait states) both
// supplies that wait and keeps the data registers allocated across it (the
// register allocator was seen reusing them in the very next instruction).
__device__ __forceinline__ void st128s(rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
    asm volatile("s_nop 1" ::"v"(v));
}
__device__ __forceinline__ void st128(rsrc_t r, uint32_t off, u32x4 v) { st128s(r, off, 0, v); }
// Non-temporal ("nt" cache policy) 16-byte store, for output written in
// whole 128-byte lines (staged probability rows, zero fills): it streams
// through L2 instead of displacing the K/V tiles other workgroups still read
// (measured: 2k x 2k D=128 non-causal prefill 170 -> 144 us). Stores of
// partial lines (the 32-byte row pieces of the MFMA layout) stay plain: with
// nt they lose L2 write combining (measured several times slower).
__device__ __forceinline__ void st128_nt(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
    asm volatile("s_nop 1" ::"v"(v));
}

// ---------------------------------------------------------------- element traits

template <typename T> struct Tr;

template <> struct Tr<__bf16> {
    static constexpr int KH = 8;  // operand elements per lane per MFMA
    using vec = bf16x8;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec cvt8(const float* x) {
        f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(f, vec);  // round to nearest even
    }
    static __device__ __forceinline__ float to_f(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }
    // Residual of the rounding hi = cvt8(x), itself rounded: x - hi is exact
    // in float32 (hi is within half a unit of x), so hi + lo carries x to
    // 16 significant bits where hi alone carries 8.
    static __device__ __forceinline__ vec lo8(const float* x, vec hi) {
        const u32x4 b = __builtin_bit_cast(u32x4, hi);
        f32x8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = b[e];
            r[2 * e] = x[2 * e] - __builtin_bit_cast(float, w << 16);
            r[2 * e + 1] = x[2 * e + 1] - __builtin_bit_cast(float, w & 0xffff0000u);
        }
        return __builtin_convertvector(r, vec);
    }
};

template <> struct Tr<_Float16> {
    static constexpr int KH = 8;
    using vec = f16x8;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ vec cvt8(const float* x) {
        f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        return __builtin_convertvector(f, vec);  // round to nearest even
    }
    static __device__ __forceinline__ float to_f(uint32_t bits16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    }
    // Residual of the rounding hi = cvt8(x), itself rounded (exact in
    // float32, as for bf16): hi + lo carries x to 22 significant bits.
    // x - hi in one mixed-precision fma per element (hi taken from its
    // packed half as a half-precision operand, times -1, plus x): the same
    // exact difference as widening hi and subtracting, in one instruction
    // instead of two.
    static __device__ __forceinline__ vec lo8(const float* x, vec hi) {
        const u32x4 b = __builtin_bit_cast(u32x4, hi);
        f32x8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = b[e];
            float d0, d1;
            asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d0) : "v"(w), "v"(x[2 * e]));
            asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d1) : "v"(w), "v"(x[2 * e + 1]));
            r[2 * e] = d0;
            r[2 * e + 1] = d1;
        }
        return __builtin_convertvector(r, vec);
    }
};

template <> struct Tr<float> {
    static constexpr int KH = 1;
    using vec = float;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// 16-byte chunk <-> operand vector
template <typename T>
__device__ __forceinline__ typename Tr<T>::vec as_vec(u32x4 x) {
    static_assert(sizeof(T) == 2, "16-byte operand vectors are 16-bit elements");
    return __builtin_bit_cast(typename Tr<T>::vec, x);
}

// ---------------------------------------------------------------- work mapping

struct Work {
    int b, hq, qblk;
};

// Workgroup ids are handed to the 8 XCDs in turn (id % 8), each XCD with its
// own L2. Remap so that an XCD receives a contiguous range of logical ids:
// the query blocks of a (batch, head), and the heads that share a KV head,
// then read K and V through the same L2. Orders (a.sched):
//  0  head-major; causal blocks of a head heaviest (latest) first;
//  1  causal: the XCD's first half of dispatches takes the heavy blocks in
//     decreasing order, its second half the light ones increasing;
//  2  causal: heaviest first over the whole grid (every head at once);
//  3  causal: each XCD takes its heads two at a time, the pair's blocks
//     interleaved heaviest first: the balance of heaviest-first order with
//     the K/V working set of two heads per L2 (measured fastest);
//  4  dispatch order, no remap: consecutive blocks run at the same time on
//     all eight XCDs, every XCD takes a share of every head (head rows:
//     each XCD then carries a share of every batch's key-padding work;
//     measured fastest, though each XCD's L2 fetches every KV head);
//  5  each XCD takes a contiguous range of heads (head sets with head rows),
//     its blocks query-block-major: all of its heads advance together, so
//     the workgroups that run at once read several heads' K/V tiles instead
//     of one, each K/V read through one XCD's L2.
__device__ __forceinline__ Work decode_block(int L, const FwdArgs& a) {
    const int nb = a.n_blocks;
    const int nfull = nb & ~7;
    const int nq = a.n_qblk;
    Work w;
    if (L < nfull && a.sched != 2 && a.sched != 4) {
        const int per = nfull >> 3;
        const int x = L & 7, i = L >> 3;
        if (a.sched == 1) {
            const int hx = per / nq;  // whole heads per XCD
            const int half = per >> 1;
            const int j = i < half ? i : i - half;
            const int head = x * hx + j % hx;
            const int r = i < half ? nq - 1 - j / hx : j / hx;
            w.b = head / a.Hq;
            w.hq = head - w.b * a.Hq;
            w.qblk = r;
            return w;
        }
        if (a.sched == 5 && per % nq == 0) {
            const int hx = per / nq;
            const int head = x * hx + i % hx, r = i / hx;
            const int hs = a.head_rows > 0 ? a.head_rows : 1;
            const int hpb = a.Hq / hs;
            w.b = head / hpb;
            w.hq = (head - w.b * hpb) * hs;
            w.qblk = a.causal ? nq - 1 - r : r;
            return w;
        }
        if (a.sched == 3 && per % (2 * nq) == 0) {
            const int g = i / (2 * nq), j = i - g * 2 * nq;
            const int head = x * (per / nq) + 2 * g + (j & 1);
            w.b = head / a.Hq;
            w.hq = head - w.b * a.Hq;
            w.qblk = nq - 1 - (j >> 1);
            return w;
        }
        L = x * per + i;
    }
    if (a.sched == 2) {
        // causal, heaviest first over the whole grid (longest-processing-time
        // order): all (batch, head) slices' last blocks, then the blocks
        // before them, ...; a slot that frees up takes the heaviest block left
        const int nbh = a.B * a.Hq;
        const int bh = L % nbh;
        w.qblk = nq - 1 - L / nbh;
        w.b = bh / a.Hq;
        w.hq = bh - w.b * a.Hq;
        return w;
    }
    const int bh = L / nq;
    const int r = L - bh * nq;
    w.qblk = a.causal ? (nq - 1 - r) : r;
    // with head rows, bh counts head sets of a.head_rows query heads (w.hq: the first)
    const int hs = a.head_rows > 0 ? a.head_rows : 1;
    const int hpb = a.Hq / hs;
    w.b = bh / hpb;
    w.hq = (bh - w.b * hpb) * hs;
    return w;
}

// ---------------------------------------------------------------- masks and scores

// Mask terms for the 16 keys lane (n, h) holds in one 32-key block starting
// at key jblk: base-2 additive terms (a bool mask gives 0 where it keeps the
// key, -inf where it removes it).
// VEC: the mask row is contiguous and 8-byte (bool) / 16-byte aligned, and
// Skv is a multiple of 8, so each run of 8 keys is one load.
template <typename T, int MASK, bool VEC>
__device__ __forceinline__ void load_mask16(const FwdArgs& a, rsrc_t mr, uint32_t row_off, int jblk, int hf,
                                            float* out) {
    constexpr int ME = MASK == MASK_BOOL ? 1 : (int)sizeof(T);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int j = jblk + 16 * c + 8 * hf;
        if constexpr (VEC) {
            const uint32_t off = pred(j < a.Skv, row_off + (uint32_t)j * ME);
            if constexpr (MASK == MASK_BOOL) {
                const u32x2 w = ld64(mr, off);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[8 * c + e] = ((w[e >> 2] >> (8 * (e & 3))) & 0xffu) ? 0.0f : -INFINITY;
            } else if constexpr (sizeof(T) == 2) {
                const u32x4 w = ld128(mr, off);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[8 * c + e] = Tr<T>::to_f((w[e >> 1] >> (16 * (e & 1))) & 0xffffu) * LOG2E;
            } else {
                const u32x4 w0 = ld128(mr, off);
                const u32x4 w1 = ld128(mr, off + 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // element to a scalar first: bit_cast of a vector element
                    // reads element 0 whatever the index (seen with this clang)
                    const uint32_t b0 = w0[e], b1 = w1[e];
                    out[8 * c + e] = __builtin_bit_cast(float, b0) * LOG2E;
                    out[8 * c + 4 + e] = __builtin_bit_cast(float, b1) * LOG2E;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = pred(j + e < a.Skv, row_off + (uint32_t)((int64_t)(j + e) * a.m_s[3] * ME));
                if constexpr (MASK == MASK_BOOL) {
                    out[8 * c + e] = __builtin_amdgcn_raw_buffer_load_b8(mr, off, 0, 0) ? 0.0f : -INFINITY;
                } else if constexpr (sizeof(T) == 2) {
                    out[8 * c + e] = Tr<T>::to_f(__builtin_amdgcn_raw_buffer_load_b16(mr, off, 0, 0)) * LOG2E;
                } else {
                    out[8 * c + e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mr, off, 0, 0)) * LOG2E;
                }
            }
        }
    }
}

// Scaled, masked scores of one S^T block in the base-2 domain; -inf where a
// key is removed (causal, mask, or past the end of the keys). `edge` says the
// block may contain keys past Skv or past this wave's causal diagonal.
template <int MASK>
__device__ __forceinline__ void scores16(const FwdArgs& a, const f32x16& acc, const float* mv, int jblk, int hf,
                                         int qi, bool edge, float* t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float x = acc[r] * a.scale_log2;
        if constexpr (MASK != MASK_NONE) x = x + mv[r];  // + 0 keeps x, + -inf removes the key
        bool drop = false;
        if (edge) {
            const int j = jblk + kk(hf, r);
            drop = drop || j >= a.Skv || (a.causal && j > qi + a.coff);
        }
        t[r] = drop ? -INFINITY : x;
    }
}

// ---------------------------------------------------------------- stores

// Eight consecutive values x[0..8) to row elements [j, j+8) (already
// converted to the row's dtype by the caller for 16-bit types).
// VEC: one (16-bit) or two (float) 16-byte stores, predicated as a whole;
// otherwise one predicated element store each.
template <typename T, bool VEC>
__device__ __forceinline__ void store8(rsrc_t r, uint32_t row_off, bool row_ok, int j, int limit, const float* x) {
    if constexpr (sizeof(T) == 2) {
        const u32x4 v = __builtin_bit_cast(u32x4, Tr<T>::cvt8(x));
        if constexpr (VEC) {
            st128(r, pred(row_ok && j < limit, row_off + (uint32_t)j * 2), v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[e >> 1] >> (16 * (e & 1))), r,
                                                      pred(row_ok && j + e < limit, row_off + (uint32_t)(j + e) * 2), 0, 0);
        }
    } else {
        if constexpr (VEC) {
            const uint32_t off = pred(row_ok && j < limit, row_off + (uint32_t)j * 4);
            st128(r, off, u32x4{__builtin_bit_cast(uint32_t, x[0]), __builtin_bit_cast(uint32_t, x[1]),
                                __builtin_bit_cast(uint32_t, x[2]), __builtin_bit_cast(uint32_t, x[3])});
            st128(r, off == OOB ? OOB : off + 16,
                  u32x4{__builtin_bit_cast(uint32_t, x[4]), __builtin_bit_cast(uint32_t, x[5]),
                        __builtin_bit_cast(uint32_t, x[6]), __builtin_bit_cast(uint32_t, x[7])});
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x[e]), r,
                                                      pred(row_ok && j + e < limit, row_off + (uint32_t)(j + e) * 4), 0, 0);
        }
    }
}

// Zero row elements [c0, c1) of rows row0 .. row0+31 (< Sq): the 64 lanes of a
// wave write 16-byte chunks (VEC) or single elements.
template <typename T, bool VEC>
__device__ __forceinline__ void zero_rows(rsrc_t r, int64_t row_stride, int row0, int Sq, int c0, int c1, int lane) {
    if (c0 >= c1) return;
    if constexpr (VEC) {
        constexpr int E = 16 / sizeof(T);
        const int nch = (c1 - c0) / E;  // c0, c1 are multiples of E here
        const int total = 32 * nch;
        for (int i = lane; i < total; i += 64) {
            const int rr = i / nch, ch = i - rr * nch;
            const int row = row0 + rr;
            st128_nt(r, pred(row < Sq, (uint32_t)((int64_t)row * row_stride * sizeof(T)) + (uint32_t)(c0 + ch * E) * sizeof(T)),
                  u32x4{0u, 0u, 0u, 0u});
        }
    } else {
        const int n = c1 - c0;
        const int total = 32 * n;
        for (int i = lane; i < total; i += 64) {
            const int rr = i / n, c = i - rr * n;
            const int row = row0 + rr;
            const uint32_t off = pred(row < Sq, (uint32_t)((int64_t)row * row_stride * sizeof(T)) + (uint32_t)(c0 + c) * sizeof(T));
            if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, r, off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b32(0u, r, off, 0, 0);
        }
    }
}

}  // namespace sdpa
