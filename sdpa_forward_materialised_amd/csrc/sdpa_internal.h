// Internal interface between the host side (validation, planning, C ABI) and
// the gfx950 kernels. Not installed; the public interface is include/sdpa_math.h.
#pragma once

#include <cstddef>
#include <cstdint>

namespace sdpa {

enum MaskKind : int { MASK_NONE = 0, MASK_BOOL = 1, MASK_ADD = 2 };
enum Dtype : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_BOOL = 3 };

// Everything a kernel needs, passed by value. Strides are in elements and
// ordered (batch, head, row); the last dim is contiguous. Mask strides cover
// the logical [B, Hq, Sq, Skv] index, 0 on broadcast dims.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;
    void* o;
    void* p;
    float* lse;
    int64_t q_s[3], k_s[3], v_s[3], o_s[3], p_s[3], l_s[3];
    int64_t m_s[4];
    int B, Hq, Hkv, Sq, Skv, group;
    int causal;
    int coff;        // causal: key j is removed for query i when j > i + coff
                     // (0 top-left; Skv - Sq bottom-right)
    int mask_vec;    // mask rows can be read with aligned vector loads
    int p_vec;       // P rows can be written with aligned 16-byte stores
    int o_vec;       // O rows likewise
    float scale_log2;  // scale * log2(e): scores live in the base-2 domain
    int n_qblk;      // query blocks per (batch, head)
    int n_blocks;    // workgroups in the grid
    int keys_per_wave;  // fused path: key range of one wave
    int fused_rg;       // fused path: 0 one row group per workgroup; else the
                        // wide variant with this many 32-row groups
    int fused_hg;       // wide variant: its row groups are fused_rg query heads
                        // of one KV group on the same 32 rows (K, V staged once)
    int fused_oseq;     // wide variant: partial outputs accumulated in turn in
                        // one LDS buffer per row group (less LDS)
    int sched;       // workgroup order (causal: 1, 2, 3; 4: dispatch order; 5: heads together), see decode_block
    int head_rows;   // two-pass, no loader wave: 0, or the number of query heads
                     // of one KV group a workgroup takes (one per compute wave,
                     // all on the same 32 rows; the mask, if any, shared by the heads)
    // Key ranges (split over workgroups): n_splits ranges of split_tiles
    // tiles (an even count) per query block; the two-pass kernels then run as
    // a statistics launch, a probability launch and an output combine, with
    // per-range row statistics (max, sum) and float32 partial O in the
    // caller's workspace: ws_ml [n_splits][B*Hq][Sq], ws_o [n_splits][B*Hq][Sq][Dv].
    int n_splits;
    int split_tiles;
    float2* ws_ml;
    float* ws_o;
    // Key ranges of the wide fused kernel (one sweep per range): each range's
    // probabilities relative to its own row maximum, float32, in
    // ws_e [B*Hq][Sq][Skv]; a combine launch scales them by the row's final
    // normaliser into P.
    float* ws_e;
    // Byte extent of one (batch, head) slice of each tensor (< 2^31); the
    // kernels address every tensor through a buffer descriptor of this size.
    uint32_t q_ext, k_ext, v_ext, o_ext, p_ext, m_ext, l_ext;
    // Dropout (kernels built with it only): a bool keep-mask over the logical
    // [B, Hq, Sq, Skv] index (strides in elements, 0 on broadcast dims); the
    // stored probability is keep * P * drop_pscale and the output product
    // takes keep * P * drop_oscale.
    const uint8_t* keep;
    int64_t kp_s[4];
    uint32_t kp_ext;
    int keep_vec;       // keep rows: 8-byte aligned, contiguous, Skv a multiple of 8
    float drop_pscale;  // 1 (explicit rule) or 1 / (1 - p) (random rule)
    float drop_oscale;  // 1 / (1 - p)
    // Packed variable-length sequences (thd != 0): B sequences whose token
    // ranges are cu_q[b] .. cu_q[b+1] of the Tq packed query tokens and
    // cu_k[b] .. cu_k[b+1] of the Tkv key tokens (device int32 arrays); Sq and
    // Skv hold the maximum lengths, the batch strides are 0, and each
    // probability row has p_cols entries (zeros past its sequence's keys).
    int thd;
    int thd_bottom_right;  // causal alignment per sequence: key j removed when j > i + Skv_b - Sq_b
    const int* cu_q;
    const int* cu_k;
    int Tq, Tkv;
    int p_cols;
};

// Backward: the forward's arguments (q, k, v, mask, lse, shapes, strides,
// causal offset, base-2 scale; o and p unused) plus the upstream gradients
// dout [B,Hq,Sq,Dv] and dprobs [B,Hq,Sq,Skv] (may be null), the outputs dq,
// dk, dv, and the per-row sum D_i = sum_j P_ij dP_ij in a float32 workspace
// [B*Hq*Sq]. Strides (batch, head, row) in elements, like FwdArgs.
struct BwdArgs {
    FwdArgs f;
    const void* dout;
    const void* dprobs;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;
    // key-side launch over query ranges (kv_splits > 1): float32 partial dk
    // and dv of each range, [range][b * Hkv + hkv][key][D] (dk, then dv),
    // summed in range order by a reduce launch
    float* ws_kv;
    int kv_splits;
    int64_t do_s[3], dp_s[3], dq_s[3], dk_s[3], dv_s[3];
    float scale;       // multiplier of Q K^T (the gradients of q and k carry it)
    int dp_vec;        // dprobs rows: aligned 16-byte loads, Skv a multiple of 8
    uint32_t do_ext, dp_ext, dq_ext, dk_ext, dv_ext;
};

// Launch configuration chosen on the host for one call.
struct Plan {
    int path;        // 1 fused, 2 two-pass
    int waves;       // waves per workgroup
    int q_rows;      // query rows per workgroup
    int n_qblk;
    int64_t grid;
    int keys_per_wave;  // fused only
    int fused_rg = 0;   // fused only: row groups of the wide variant (0: the one-group kernel)
    int fused_hg = 0;   // wide variant: row groups are query heads of one KV group
    int fused_oseq = 0; // wide variant: partial outputs accumulated in turn (less LDS)
    int64_t tiles_per_bh;
    int64_t tiles_64;
    int head_rows = 0;    // two-pass: query heads per workgroup on shared rows (0: one head)
    int n_splits = 1;     // key ranges per query block (with a workspace)
    int split_tiles = 0;  // two-pass: kernel tiles per key range (even)
    // n_splits > 1 on the fused path: key ranges of the wide kernel, one sweep
    // each (keys_per_wave * waves keys per range), then a combine launch
};

// Kernel launchers, one translation unit per dtype. `vec` selects the
// variant with 16-byte row stores and vector mask loads (rows aligned, Skv a
// multiple of 8, mask contiguous in its last dim); the other variant handles
// any layout element by element. Return a hipError_t as int.
// `drop`: the dropout variant (two compute waves and a loader wave only).
int launch_twopass_f32(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream);
int launch_twopass_f16(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream);
int launch_twopass_bf16(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream);
int launch_fused(int dtype, int D, int mask_kind, int waves, bool vec, const FwdArgs& a, void* stream);
// Backward launches (query-side kernel, then key/value-side kernel) on the
// stream; hipError_t as int.
int launch_backward(int dtype, int D, int mask_kind, const BwdArgs& a, void* stream);
// Whether the two-pass kernel can run four compute waves without a loader
// wave (16-byte layouts) for this head dim and mask kind.
bool twopass_nl_ok_f32(int D, int mask_kind);
bool twopass_nl_ok_f16(int D, int mask_kind);
bool twopass_nl_ok_bf16(int D, int mask_kind);

// Bytes of the per-device static scratch behind sdpa_math_fwd_noalloc (the
// key-range workspace: per range and query row a (max, sum) pair and a
// float32 partial output row). Must match SDPA_MATH_NOALLOC_SCRATCH_BYTES.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(32) << 20;
// Device address of the current device's static scratch (hipError_t as int).
int static_scratch(void** ptr);

// Largest key range the fused path keeps on chip per wave (scores held in
// registers: 32 rows x keys / 64 lanes floats per lane), by head dim.
constexpr int FUSED_MAX_KEYS_PER_WAVE = 256;       // D = 32, 64
constexpr int FUSED_MAX_KEYS_PER_WAVE_D128 = 128;  // D = 128
constexpr int FUSED_MAX_WAVES = 8;
// Wide fused variant: keys per wave, and the LDS it may take for the staged V
// rows of all its keys (or the partial outputs), plus the row statistics.
// Keys per wave: D = 32, 64: 320; D = 128: 160 (float32: 128).
constexpr int fused_wide_max_keys(int dtype, int D) { return D == 128 ? (dtype == DT_F32 ? 128 : 160) : 320; }
constexpr int FUSED_LDS_MAX = 160 * 1024;
// Bytes of dynamic LDS of the wide variant for `nw` waves in `rg` row groups
// staging `vrows` V rows (`oseq`: partial outputs accumulated in turn).
inline int fused_wide_lds_bytes_rt(int dtype, int D, int nw, int rg, int vrows, bool oseq) {
    const int esz = dtype == DT_F32 ? 4 : 2;
    const int v = vrows * D * esz, o = nw == rg ? 0 : (oseq ? rg : nw) * 32 * (D + 4) * 4;
    return (v > o ? v : o) + 2 * nw * 32 * 4;
}
constexpr int TILE_N = 64;  // keys per score tile
// Most key ranges of one call on the wide kernel (the combine keeps a scale per range in LDS).
constexpr int RANGE_MAX = 4096;

}  // namespace sdpa
