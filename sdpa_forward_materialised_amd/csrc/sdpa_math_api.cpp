// Host side of the sdpa_math C ABI: argument validation, shape resolution,
// the tile-count path choice and the kernel launch. No device memory is
// allocated here, nothing is synchronised and no device data is read.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "sdpa_internal.h"
#include "sdpa_math.h"

namespace {

thread_local std::string g_last_error;

sdpa_status_t fail(sdpa_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

int64_t elt_size(int dtype) {
    switch (dtype) {
        case SDPA_F32: return 4;
        case SDPA_F16:
        case SDPA_BF16: return 2;
        case SDPA_BOOL: return 1;
        default: return 0;
    }
}

const char* dtype_name(int dtype) {
    switch (dtype) {
        case SDPA_F32: return "f32";
        case SDPA_F16: return "f16";
        case SDPA_BF16: return "bf16";
        case SDPA_BOOL: return "bool";
        default: return "?";
    }
}

int64_t numel(const sdpa_tensor_t* t) {
    int64_t n = 1;
    for (int d = 0; d < t->ndim; ++d) n *= t->sizes[d];
    return n;
}

// Effective stride: a size-1 dim never advances, whatever stride it carries.
int64_t eff_stride(const sdpa_tensor_t* t, int d) { return t->sizes[d] == 1 ? 0 : t->strides[d]; }

// True when every row start (all dims but the last) is `align`-byte aligned.
bool rows_aligned(const sdpa_tensor_t* t, int64_t align) {
    const int64_t es = elt_size(t->dtype);
    if (reinterpret_cast<uintptr_t>(t->data) % align) return false;
    for (int d = 0; d + 1 < t->ndim; ++d)
        if ((eff_stride(t, d) * es) % align) return false;
    return true;
}

struct Shape {
    int64_t B, Hq, Hkv, Sq, Skv, D, Dv;
    int dtype;
    int mask_kind;
    bool mask_head_shared;  // no mask, or one that every query head shares (size 1 or stride 0)
};

sdpa_status_t check_tensor(const sdpa_tensor_t* t, const char* name, int ndim) {
    if (!t) return fail(SDPA_ERR_INVALID_ARG, "%s is NULL", name);
    if (t->ndim != ndim) return fail(SDPA_ERR_INVALID_ARG, "%s must have %d dims, got %d", name, ndim, t->ndim);
    for (int d = 0; d < ndim; ++d)
        if (t->sizes[d] < 0) return fail(SDPA_ERR_INVALID_ARG, "%s has a negative size", name);
    if (elt_size(t->dtype) == 0) return fail(SDPA_ERR_INVALID_ARG, "%s has an unknown dtype %d", name, t->dtype);
    if (numel(t) > 0 && t->data == nullptr) return fail(SDPA_ERR_INVALID_ARG, "%s has no data pointer", name);
    if (numel(t) > 0 && t->sizes[ndim - 1] > 1 && t->strides[ndim - 1] != 1)
        return fail(SDPA_ERR_UNSUPPORTED, "%s must be contiguous in its last dim (stride %lld)", name,
                    (long long)t->strides[ndim - 1]);
    return SDPA_OK;
}

sdpa_status_t check_dims(const sdpa_tensor_t* t, const char* name, const int64_t* want, int ndim) {
    for (int d = 0; d < ndim; ++d)
        if (t->sizes[d] != want[d]) {
            return fail(SDPA_ERR_INVALID_ARG, "%s dim %d is %lld, expected %lld", name, d, (long long)t->sizes[d],
                        (long long)want[d]);
        }
    return SDPA_OK;
}

sdpa_status_t validate_inputs(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                              const sdpa_tensor_t* mask, int is_causal, int enable_gqa, Shape* sh) {
    sdpa_status_t st;
    if ((st = check_tensor(q, "q", 4)) || (st = check_tensor(k, "k", 4)) || (st = check_tensor(v, "v", 4)))
        return st;
    if (q->dtype != SDPA_F32 && q->dtype != SDPA_F16 && q->dtype != SDPA_BF16)
        return fail(SDPA_ERR_INVALID_ARG, "q dtype %s is not f32, f16 or bf16", dtype_name(q->dtype));
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(SDPA_ERR_INVALID_ARG, "q, k, v dtypes differ (%s, %s, %s)", dtype_name(q->dtype),
                    dtype_name(k->dtype), dtype_name(v->dtype));
    sh->B = q->sizes[0];
    sh->Hq = q->sizes[1];
    sh->Sq = q->sizes[2];
    sh->D = q->sizes[3];
    sh->Hkv = k->sizes[1];
    sh->Skv = k->sizes[2];
    sh->Dv = v->sizes[3];
    sh->dtype = q->dtype;
    if (k->sizes[0] != sh->B || v->sizes[0] != sh->B)
        return fail(SDPA_ERR_INVALID_ARG, "batch sizes differ: q %lld, k %lld, v %lld", (long long)sh->B,
                    (long long)k->sizes[0], (long long)v->sizes[0]);
    if (v->sizes[1] != sh->Hkv || v->sizes[2] != sh->Skv)
        return fail(SDPA_ERR_INVALID_ARG, "k and v disagree on heads or length");
    if (k->sizes[3] != sh->D)
        return fail(SDPA_ERR_INVALID_ARG, "q and k head dims differ (%lld vs %lld)", (long long)sh->D,
                    (long long)k->sizes[3]);
    if (sh->Hkv <= 0 || sh->Hq % sh->Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARG, "query heads (%lld) are not a multiple of key/value heads (%lld)",
                    (long long)sh->Hq, (long long)sh->Hkv);
    if (sh->Hq != sh->Hkv && !enable_gqa)
        return fail(SDPA_ERR_INVALID_ARG, "Hq (%lld) != Hkv (%lld) needs enable_gqa", (long long)sh->Hq,
                    (long long)sh->Hkv);
    if (is_causal < 0 || is_causal > 2)
        return fail(SDPA_ERR_INVALID_ARG, "is_causal must be 0 (none), 1 (top-left) or 2 (bottom-right), got %d",
                    is_causal);
    sh->mask_kind = sdpa::MASK_NONE;
    sh->mask_head_shared = !mask || mask->sizes[1] == 1 || mask->strides[1] == 0;
    if (mask) {
        if (is_causal) return fail(SDPA_ERR_INVALID_ARG, "is_causal and an explicit mask are mutually exclusive");
        if (mask->ndim != 4) return fail(SDPA_ERR_INVALID_ARG, "mask must be passed with 4 dims (right-aligned)");
        for (int d = 0; d < 4; ++d)
            if (mask->sizes[d] < 0) return fail(SDPA_ERR_INVALID_ARG, "mask has a negative size");
        const int64_t full[4] = {sh->B, sh->Hq, sh->Sq, sh->Skv};
        for (int d = 0; d < 4; ++d)
            if (mask->sizes[d] != 1 && mask->sizes[d] != full[d])
                return fail(SDPA_ERR_INVALID_ARG, "mask dim %d (%lld) does not broadcast to %lld", d,
                            (long long)mask->sizes[d], (long long)full[d]);
        if (mask->dtype == SDPA_BOOL) sh->mask_kind = sdpa::MASK_BOOL;
        else if (mask->dtype == q->dtype) sh->mask_kind = sdpa::MASK_ADD;
        else
            return fail(SDPA_ERR_INVALID_ARG, "mask dtype %s must be bool or the query dtype %s",
                        dtype_name(mask->dtype), dtype_name(q->dtype));
        if (numel(mask) > 0 && !mask->data) return fail(SDPA_ERR_INVALID_ARG, "mask has no data pointer");
    }
    if (sh->Sq > INT32_MAX || sh->Skv > INT32_MAX || sh->B > INT32_MAX || sh->Hq > INT32_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond 2^31 are not supported");
    if (sh->D != 32 && sh->D != 64 && sh->D != 128)
        return fail(SDPA_ERR_UNSUPPORTED, "head dim %lld is not implemented (32, 64, 128)", (long long)sh->D);
    if (sh->Dv != sh->D)
        return fail(SDPA_ERR_UNSUPPORTED, "value head dim %lld != query head dim %lld is not implemented",
                    (long long)sh->Dv, (long long)sh->D);
    const sdpa_tensor_t* in[3] = {q, k, v};
    const char* names[3] = {"q", "k", "v"};
    for (int i = 0; i < 3; ++i)
        if (numel(in[i]) > 0 && !rows_aligned(in[i], 16))
            return fail(SDPA_ERR_UNSUPPORTED, "%s needs a 16-byte aligned base and 16-byte multiple strides", names[i]);
    return SDPA_OK;
}

sdpa_status_t validate_outputs(const Shape& sh, const sdpa_tensor_t* out, const sdpa_tensor_t* probs,
                               const sdpa_tensor_t* lse) {
    sdpa_status_t st;
    if ((st = check_tensor(out, "out", 4)) || (st = check_tensor(probs, "probs", 4)) ||
        (st = check_tensor(lse, "lse", 3)))
        return st;
    if (out->dtype != sh.dtype || probs->dtype != sh.dtype)
        return fail(SDPA_ERR_INVALID_ARG, "out and probs must have the query dtype %s", dtype_name(sh.dtype));
    if (lse->dtype != SDPA_F32) return fail(SDPA_ERR_INVALID_ARG, "lse must be f32");
    const int64_t wo[4] = {sh.B, sh.Hq, sh.Sq, sh.Dv};
    const int64_t wp[4] = {sh.B, sh.Hq, sh.Sq, sh.Skv};
    const int64_t wl[3] = {sh.B, sh.Hq, sh.Sq};
    if ((st = check_dims(out, "out", wo, 4)) || (st = check_dims(probs, "probs", wp, 4)) ||
        (st = check_dims(lse, "lse", wl, 3)))
        return st;
    return SDPA_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Causal diagonal offset: key j is removed for query i when j > i + offset
// (is_causal 1: top-left, offset 0; 2: bottom-right, the alignment of a query
// chunk against a longer key cache, offset Skv - Sq).
int64_t causal_offset(const Shape& sh, int is_causal) { return is_causal == 2 ? sh.Skv - sh.Sq : 0; }

// Score tiles one (batch, head) processes with `rows` query rows per block
// and 64 keys per tile, after causal truncation (key j removed for query i
// when j > i + coff: coff 0 top-left, Skv - Sq bottom-right).
int64_t count_tiles(int64_t Sq, int64_t Skv, bool causal, int64_t rows, int64_t coff = 0) {
    const int64_t ktiles = cdiv(Skv, sdpa::TILE_N);
    if (!causal) return cdiv(Sq, rows) * ktiles;
    int64_t total = 0;
    for (int64_t r0 = 0; r0 < Sq; r0 += rows) {
        const int64_t last = std::min(Sq, r0 + rows) + coff;  // keys j < last are reachable
        total += cdiv(std::max<int64_t>(0, std::min(Skv, last)), sdpa::TILE_N);
    }
    return total;
}

// Fused-path switch. The FlagOS-OP page switches on the causal-truncated
// count of 64x64 score tiles per (batch, head) and settled on 56 for its
// hardware. Measured on MI355X (kernel times of both paths over D 64/128,
// causal and not, Sq 32..1024, Skv 128..2048), the tile count alone picks
// the fused kernel where it loses: it re-reads K and V for every 32-row
// block, while the two-pass kernel shares them over 96-128 rows and only
// runs out of parallelism when the query range is short; a non-causal call
// with few keys per row gives the fused kernel too little to hide its
// latencies. The switch is therefore: fused iff Sq <= 128 rows, at most 64
// tiles per (batch, head), and (causal or Skv >= 512) -- 0.5 % above the
// per-shape best on the sweep (worst shape 1.11x); tile count alone at its
// best threshold is 6 % off and up to 1.4x.
constexpr int64_t kFusedMaxTiles64 = 64;
constexpr int64_t kFusedMaxRows = 128;
constexpr int64_t kFusedMinKeysNonCausal = 512;

int env_path() {
    const char* e = std::getenv("SDPA_MATH_PATH");
    if (!e) return SDPA_PATH_AUTO;
    if (!std::strcmp(e, "fused")) return SDPA_PATH_FUSED;
    if (!std::strcmp(e, "twopass")) return SDPA_PATH_TWOPASS;
    return SDPA_PATH_AUTO;
}

int64_t env_max_tiles() {
    const char* e = std::getenv("SDPA_MATH_FUSED_MAX_TILES");
    if (!e || !*e) return kFusedMaxTiles64;
    return std::strtoll(e, nullptr, 10);
}

int64_t env_min_keys() {
    const char* e = std::getenv("SDPA_MATH_FUSED_MIN_KEYS");
    if (!e || !*e) return kFusedMinKeysNonCausal;
    return std::strtoll(e, nullptr, 10);
}

int64_t env_max_rows() {
    const char* e = std::getenv("SDPA_MATH_FUSED_MAX_ROWS");
    if (!e || !*e) return kFusedMaxRows;
    return std::strtoll(e, nullptr, 10);
}

// Fused path: one workgroup = 32 query rows, keys split over up to 8 waves,
// each keeping at most the per-head-dim limit of scores in registers. Waves
// are added until a wave holds at most 128 keys (fewer registers, more waves
// in flight) or the wave count is at its maximum.
bool fused_config(const Shape& sh, bool causal, int64_t coff, int* waves, int* keys_per_wave) {
    const int64_t keys = causal ? std::min(sh.Skv, sh.Sq + coff) : sh.Skv;  // the last row's keys
    if (keys <= 0) return false;
    const int64_t limit = sh.D == 128 ? sdpa::FUSED_MAX_KEYS_PER_WAVE_D128 : sdpa::FUSED_MAX_KEYS_PER_WAVE;
    for (int w = 1; w <= sdpa::FUSED_MAX_WAVES; w *= 2) {
        const int64_t kpw = cdiv(cdiv(keys, w), 32) * 32;
        if (kpw <= std::min<int64_t>(limit, 128) || (w == sdpa::FUSED_MAX_WAVES && kpw <= limit)) {
            *waves = w;
            *keys_per_wave = (int)kpw;
            return true;
        }
    }
    return false;
}

// Wide fused variant: workgroups of rg row groups of 32 rows x kg key groups
// (rg * kg <= 8 waves), the K, then V, rows of all their keys staged in LDS.
// rg: the largest of 4, 2, 1 that still gives a workgroup per CU (256); kg:
// the fewest key groups whose per-wave key range and staged rows fit, then
// doubled while a wave holds more than 128 keys and wave slots are left
// (more waves in flight: measured faster for 32- and 64-row calls).
// SDPA_MATH_FUSED_WIDE=0 keeps the fused path on its one-row-group kernel;
// =1 makes the fused path take the wide variant only (an error where it
// cannot take the shape).
bool fused_wide_config(const Shape& sh, bool causal, int64_t coff, int* waves, int* keys_per_wave, int* rg_out) {
    if (const char* e = std::getenv("SDPA_MATH_FUSED_WIDE"))
        if (!std::strcmp(e, "0")) return false;
    const int64_t keys = causal ? std::min(sh.Skv, sh.Sq + coff) : sh.Skv;  // the last row's keys
    if (keys <= 0) return false;
    const int64_t n32 = cdiv(sh.Sq, 32), bh = sh.B * sh.Hq;
    const int dt = sh.dtype == SDPA_F32 ? sdpa::DT_F32 : sdpa::DT_F16;
    const int64_t limit = sdpa::fused_wide_max_keys(dt, (int)sh.D);
    for (int rg = 4; rg >= 1; rg /= 2) {
        if (rg > 1 && (rg > n32 || bh * cdiv(n32, rg) < 256)) continue;
        for (int kg = 1; rg * kg <= sdpa::FUSED_MAX_WAVES; kg *= 2) {
            const int64_t kpw = cdiv(cdiv(keys, kg), 32) * 32;
            if (kpw > limit) continue;
            if (sdpa::fused_wide_lds_bytes_rt(dt, (int)sh.D, rg * kg, rg, (int)(kg * kpw), false) > sdpa::FUSED_LDS_MAX) continue;
            int k2 = kg;
            int64_t kp2 = kpw;
            while (kp2 > 128 && rg * k2 * 2 <= sdpa::FUSED_MAX_WAVES) {
                const int64_t nk = cdiv(cdiv(keys, 2 * k2), 32) * 32;
                if (sdpa::fused_wide_lds_bytes_rt(dt, (int)sh.D, rg * 2 * k2, rg, (int)(2 * k2 * nk), false) > sdpa::FUSED_LDS_MAX)
                    break;
                k2 *= 2;
                kp2 = nk;
            }
            *waves = rg * k2;
            *keys_per_wave = (int)kp2;
            *rg_out = rg;
            return true;
        }
    }
    return false;
}

// True when the 16-byte variant of the two-pass kernel can run: probability
// and output rows 16-byte aligned (null: the default dense outputs), Skv a
// multiple of 8, and a mask (if any) contiguous along the keys with 16-byte
// aligned rows and whole 16-byte chunks.
bool staged_layout(const Shape& sh, const sdpa_tensor_t* mask, const sdpa_tensor_t* out,
                   const sdpa_tensor_t* probs) {
    if (sh.Skv % 8) return false;
    if (out && !rows_aligned(out, 16)) return false;
    if (probs && !rows_aligned(probs, 16)) return false;
    if (mask) {
        const int64_t me = sh.mask_kind == sdpa::MASK_BOOL ? 1 : elt_size(sh.dtype);
        if (eff_stride(mask, 3) != 1 || !rows_aligned(mask, 16) || sh.Skv % (16 / me)) return false;
    }
    return true;
}

// Key ranges for short grids over long keys (two-pass, loader-wave kernels,
// 16-byte layouts): with fewer than 256 blocks of 64 query rows and at least
// 32 key tiles in the heaviest block, its keys are split into ranges of an
// even number (at least 16) of tiles, towards 512 workgroups. Each workgroup
// pays a fixed start-up in each of the two launches, so shorter ranges or
// fuller grids lose (measured on MI355X, bf16: 4x8 heads, 1 query, 32768 keys
// 1003 -> 154 us; 1x32 heads, 16 queries, 16384 keys 375 -> 78 us; 2x16
// heads, 64 queries, 8192 keys at D = 64 136 -> 36 us; 8x8 heads, 32
// queries, 4096 keys 101 -> 43 us; but 100 queries x 1152 keys with 16x8
// heads 32 -> 43 us and a 512-query chunk against 2048 keys 48 -> 50 us).
// SDPA_MATH_SPLITS=n forces n ranges (1: none).
void split_plan(const Shape& sh, bool causal, int64_t coff, int* n_splits, int* split_tiles) {
    *n_splits = 1;
    *split_tiles = 0;
    const int64_t tn = sh.mask_kind == sdpa::MASK_BOOL ? 32 : 64;  // the kernels' keys per tile
    const int64_t keys = causal ? std::max<int64_t>(0, std::min(sh.Skv, sh.Sq + coff)) : sh.Skv;
    const int64_t max_tiles = cdiv(keys, tn);
    const int64_t blocks = sh.B * sh.Hq * cdiv(sh.Sq, 64);
    int64_t want = 1;
    if (blocks < 256 && max_tiles >= 32) want = std::min(cdiv(512, blocks), max_tiles / 16);
    if (const char* e = std::getenv("SDPA_MATH_SPLITS")) want = std::max<int64_t>(1, std::atoll(e));
    if (want < 2 || max_tiles < 2) return;
    int64_t per = cdiv(max_tiles, want);
    per += per & 1;
    const int64_t n = cdiv(max_tiles, per);
    if (n < 2) return;
    *n_splits = (int)n;
    *split_tiles = (int)per;
}

// Workspace bytes of a split plan: per range and row the (max, sum) pair,
// then (256-byte aligned) the float32 partial O.
size_t split_ws_ml_bytes(const Shape& sh, int n_splits) { return (size_t)n_splits * sh.B * sh.Hq * sh.Sq * 8; }
size_t split_ws_bytes(const Shape& sh, int n_splits) {
    if (n_splits <= 1) return 0;
    const size_t ml = (split_ws_ml_bytes(sh, n_splits) + 255) / 256 * 256;
    return ml + (size_t)n_splits * sh.B * sh.Hq * sh.Sq * sh.Dv * 4;
}
// Key ranges of the wide kernel add (256-byte aligned) every row's float32
// probabilities relative to its range's maximum.
size_t plan_ws_e_offset(const Shape& sh, int n_splits) { return (split_ws_bytes(sh, n_splits) + 255) / 256 * 256; }
size_t plan_ws_bytes(const Shape& sh, const sdpa::Plan& p) {
    if (p.n_splits <= 1) return 0;
    if (p.path != SDPA_PATH_FUSED) return split_ws_bytes(sh, p.n_splits);
    return plan_ws_e_offset(sh, p.n_splits) + (size_t)sh.B * sh.Hq * sh.Sq * sh.Skv * 4;
}

// One-sweep key ranges on the wide fused kernel, for few query rows against
// many keys: each workgroup scores one range of R keys (K staged in LDS, then
// V) once, and writes its probabilities relative to its own row maximum as
// float32, its rows' (max, sum) and its float32 partial O; a combine launch
// scales each range by 2^(max_r - lse2) into P and O. K and V are read once
// (the two-pass split reads K in both launches) at the price of the float32
// probabilities written and read back: 8 bytes per probability against the
// D * element-size bytes of the K row re-read per key and KV head. Measured
// (bf16 / f16, D = 64 and 128, 1 to 16 query rows, 8192 to 65536 keys) the
// ranges win where those 8 bytes times the query rows stay within a quarter
// of the K row (one or four query rows: 20-30 % faster) and lose at half of
// it (8 and 16 rows: 5-8 % slower): taken where 32 * Sq <= D * element size.
// Ungrouped heads: one row group of 32 rows and 4 key groups per workgroup,
// R = 64 KB of K rows: 256 keys at D = 128 (16-bit; 128 for float32), 512 at
// D = 64, 1024 at D = 32, so that two workgroups share a CU (one query row x
// 32768 keys, bf16, D = 128, 32 heads: 118 us, against 134 with 512-key
// ranges of 8 waves, one workgroup per CU, and 156 for the two-pass split).
// Grouped heads: the group's query heads (up to 8) are the row groups of one
// workgroup, which stages each range's K and V rows once for all of them, one
// wave per head over the range's keys (R = the most one wave holds: 160 at
// D = 128, 320 at D = 64): one query row x 32768 keys, bf16, D = 128, 2 x 32
// heads on 8 KV heads 92 us against 124 with two key groups of 128 keys and
// 133 for the two-pass split; 4 x 16 on 8: 139 against 199; 64 on 8: 96
// against 133.
// SDPA_MATH_RANGES=0 turns them off, =1 takes them wherever they fit (any
// row count); SDPA_MATH_RANGE_KEYS=R and SDPA_MATH_RANGE_WAVES=KG override.
bool range_config(const Shape& sh, bool causal, int64_t coff, int* waves, int* keys_per_wave, int* n_ranges,
                  int* rg_out) {
    const int64_t keys = causal ? std::max<int64_t>(0, std::min(sh.Skv, sh.Sq + coff)) : sh.Skv;
    const int dt = sh.dtype == SDPA_F32 ? sdpa::DT_F32 : sdpa::DT_F16;
    const int64_t es = elt_size(sh.dtype);
    const int64_t group = sh.Hq / sh.Hkv;
    // grouped heads: the group's heads (up to 8) are the row groups
    const int64_t rg = group <= sdpa::FUSED_MAX_WAVES ? group : group % sdpa::FUSED_MAX_WAVES == 0 ? sdpa::FUSED_MAX_WAVES : 0;
    if (rg == 0) return false;
    int64_t kg = rg > 1 ? 1 : 4;
    if (const char* e = std::getenv("SDPA_MATH_RANGE_WAVES")) kg = std::atoll(e);
    if (kg < 1 || rg * kg > sdpa::FUSED_MAX_WAVES) return false;
    const int64_t max_kpw = sdpa::fused_wide_max_keys(dt, (int)sh.D);
    int64_t R = rg > 1 ? max_kpw : std::min<int64_t>((64 * 1024) / (sh.D * es), kg * max_kpw) / (32 * kg) * (32 * kg);
    if (const char* e = std::getenv("SDPA_MATH_RANGE_KEYS")) R = std::atoll(e);
    if (R < 32 * kg || R % (32 * kg)) return false;
    const int64_t kpw = R / kg;
    // head row groups accumulate their partial outputs in turn (one LDS buffer
    // per row group), which keeps two workgroups per CU
    if (kpw > max_kpw ||
        sdpa::fused_wide_lds_bytes_rt(dt, (int)sh.D, (int)(rg * kg), (int)rg, (int)R, rg > 1) > sdpa::FUSED_LDS_MAX)
        return false;
    // one (batch, head) slice of the float32 probabilities must stay under 1 GiB
    if (sh.Sq * sh.Skv * 4 >= (int64_t(1) << 30) || keys <= 0) return false;
    if (cdiv(keys, R) > sdpa::RANGE_MAX) return false;
    *waves = (int)(rg * kg);
    *keys_per_wave = (int)kpw;
    *n_ranges = (int)cdiv(keys, R);
    *rg_out = (int)rg;
    return true;
}

sdpa_status_t make_plan(const Shape& sh, bool causal, int64_t coff, int forced, bool vec, sdpa::Plan* p,
                        bool allow_split = false, bool allow_ranges = true) {
    p->tiles_64 = count_tiles(sh.Sq, sh.Skv, causal, 64, coff);
    int fw = 0, fk = 0, frg = 0;
    int ww = 0, wk = 0, wrg = 0;
    const bool wide_ok = fused_wide_config(sh, causal, coff, &ww, &wk, &wrg);
    const bool fused_ok = fused_config(sh, causal, coff, &fw, &fk) || wide_ok;
    if (wide_ok) {
        fw = ww;
        fk = wk;
        frg = wrg;
    }
    int path = forced;
    if (path == SDPA_PATH_AUTO) path = env_path();
    const bool auto_path = path == SDPA_PATH_AUTO;
    // An additive mask over more than 64 query rows goes to the two-pass path
    // (it stages the mask tiles in LDS; measured: fp16, 16 x 8 heads, Sq 100
    // and 128, Skv 512 / 1152 / 2048, D = 64: equal or up to 9 % faster; with
    // a bool mask the fused path stays faster, by up to 2.5x).
    const bool add_rows = sh.mask_kind == sdpa::MASK_ADD && sh.Sq > 64;
    // Where the wide variant can take the shape it replaces that rule: with a
    // mask (read once instead of once per sweep) from 512 keys and up to 256
    // query rows, without one from 1024 keys and up to 128 rows (measured,
    // fp16, 16 x 8 heads, Sq 32..256, Skv 256..2048, D 64 / 128: e.g. 100
    // queries x 1152 keys, D 64, additive mask 30 vs 39 us; bool mask, 256 x
    // 1152 55 vs 68 us; no mask, 128 x 512 19 vs 18 us, left to two-pass).
    const bool masked = sh.mask_kind != sdpa::MASK_NONE;
    const bool wide_pick = wide_ok && !causal && sh.Skv >= (masked ? 512 : 1024) && sh.Sq <= (masked ? 256 : 128);
    // (causal calls keep the tile-count rule whichever kernel takes them)
    const bool tile_rule = fused_ok && p->tiles_64 <= env_max_tiles() && sh.Sq <= env_max_rows() &&
                           (causal || sh.Skv >= env_min_keys()) && !add_rows;
    if (path == SDPA_PATH_AUTO)
        path = (wide_ok && !causal ? wide_pick : tile_rule) ? SDPA_PATH_FUSED : SDPA_PATH_TWOPASS;
    if (path == SDPA_PATH_FUSED && !wide_ok) {
        const char* e = std::getenv("SDPA_MATH_FUSED_WIDE");
        if (e && !std::strcmp(e, "1"))
            return fail(SDPA_ERR_UNSUPPORTED, "the wide fused variant cannot take this shape (SDPA_MATH_FUSED_WIDE=1)");
    }
    if (path == SDPA_PATH_FUSED && !fused_ok)
        return fail(SDPA_ERR_UNSUPPORTED, "the fused path cannot take this shape (more than %d keys per wave x %d waves)",
                    sh.D == 128 ? sdpa::FUSED_MAX_KEYS_PER_WAVE_D128 : sdpa::FUSED_MAX_KEYS_PER_WAVE,
                    sdpa::FUSED_MAX_WAVES);
    p->path = path;
    if (path == SDPA_PATH_FUSED) {
        p->waves = fw;
        p->keys_per_wave = fk;
        p->fused_rg = frg;
        p->q_rows = 32 * (frg > 0 ? frg : 1);
    } else {
        // Workgroups of four waves take one wave slot per SIMD, so two of
        // them share a CU with the SIMDs evenly loaded (a five-wave group
        // takes two slots per SIMD and runs alone). Preferred: four compute
        // waves that share the tile loads themselves (16-byte layouts, when
        // their staged probability tiles fit in LDS); else three compute
        // waves plus a loader wave. Two compute waves when that leaves fewer
        // than one workgroup per CU (a 1024-row causal prefill at D = 64,
        // 352 blocks, runs 7 % faster on three: measured); float32 at D = 128
        // takes two (its tiles are twice as large). Causal calls keep the
        // 96-row blocks: their work per block grows with the block index,
        // and with 128-row blocks the grid no longer has enough blocks to
        // balance the CUs (measured slower).
        const int64_t bh = sh.B * sh.Hq;
        const bool nl_ok = vec && (sh.dtype == SDPA_F32    ? sdpa::twopass_nl_ok_f32((int)sh.D, sh.mask_kind)
                                   : sh.dtype == SDPA_F16 ? sdpa::twopass_nl_ok_f16((int)sh.D, sh.mask_kind)
                                                          : sdpa::twopass_nl_ok_bf16((int)sh.D, sh.mask_kind));
        if (nl_ok && !causal && bh * cdiv(sh.Sq, 128) >= 512) p->waves = 4;
        else p->waves = (bh * cdiv(sh.Sq, 96) >= 256) ? 3 : 2;
        // 96-row blocks that leave more than a quarter of their rows empty
        // (Sq = 100 or 128, say) lose to 64-row blocks (measured 4-10 %)
        if (p->waves == 3 && 4 * (cdiv(sh.Sq, 96) * 96 - sh.Sq) > cdiv(sh.Sq, 96) * 96 &&
            cdiv(sh.Sq, 64) * 64 - sh.Sq < cdiv(sh.Sq, 96) * 96 - sh.Sq)
            p->waves = 2;
        if (const char* e = std::getenv("SDPA_MATH_TP_WAVES")) {
            const int wv = std::atoi(e);
            if (wv == 2 || wv == 3 || (wv == 4 && nl_ok)) p->waves = wv;
        }
        if ((sh.dtype == SDPA_F32 && sh.D == 128 && p->waves == 3) || !vec) p->waves = 2;
        p->keys_per_wave = 0;
        if (allow_split && vec && p->waves != 4) {
            split_plan(sh, causal, coff, &p->n_splits, &p->split_tiles);
            if (p->n_splits > 1) p->waves = 2;  // key ranges run on the two-wave loader kernel
        }
        p->q_rows = 32 * p->waves;
        // Head rows: a grouped-head call on the four-wave kernel without a
        // loader wave gives each workgroup four query heads of one KV group
        // on 32 shared rows (one head per wave) instead of 128 rows of one
        // head: the same K/V tile loads per workgroup, a quarter of the mask
        // rows when the heads share the mask (measured: GQA key padding, fp16,
        // 4 x 32 heads on 8, 1024 x 1024, D = 128: 176.3 -> 165.3 us with
        // the blocks in dispatch order, 170.2 head-major per XCD).
        // SDPA_MATH_HEAD_ROWS=0 turns it off.
        const char* hr = std::getenv("SDPA_MATH_HEAD_ROWS");
        if (p->waves == 4 && !causal && (sh.Hq / sh.Hkv) % 4 == 0 && sh.mask_head_shared && !(hr && *hr == '0')) {
            p->head_rows = 4;
            p->q_rows = 32;
        }
    }
    // one-sweep key ranges on the wide kernel (range_config) for one to four
    // query rows, in place of the two-pass kernel (split or not) and of the
    // one-row-group fused kernel: K and V read once, the heads of a KV group
    // in one workgroup. Batched decode, measured (bf16, D = 128, one query
    // row, 16 x 32 heads on 8 KV heads): 1024 keys 38.8 -> 33.7 us (from the
    // one-row-group kernel), 2048 keys 93.7 -> 52.2, 4096 keys 179 -> 89 (from
    // two-pass); 16 x 32 ungrouped heads, 2048 keys 150 -> 118; four query rows
    // at D = 64 the same within noise. A call the whole-call wide kernel takes
    // keeps it.
    if (allow_split && allow_ranges && vec && auto_path) {
        const char* re = std::getenv("SDPA_MATH_RANGES");
        // (a forced two-pass range count, SDPA_MATH_SPLITS, keeps the two-pass ranges)
        const bool force = re && *re == '1', off = (re && *re == '0') || (!force && std::getenv("SDPA_MATH_SPLITS"));
        const bool fewer_bytes = 32 * sh.Sq <= sh.D * elt_size(sh.dtype);
        const bool whole_wide = p->path == SDPA_PATH_FUSED && p->fused_rg > 0;
        int rw = 0, rk = 0, rn = 0, rrg = 0;
        if (!off && (force || (fewer_bytes && !whole_wide)) &&
            range_config(sh, causal, coff, &rw, &rk, &rn, &rrg) && rn >= 2) {
            p->path = SDPA_PATH_FUSED;
            p->waves = rw;
            p->keys_per_wave = rk;
            p->head_rows = 0;
            p->fused_rg = rrg;
            p->fused_hg = sh.Hq != sh.Hkv;
            p->fused_oseq = rrg > 1;
            p->q_rows = 32;
            p->n_splits = rn;
            p->split_tiles = 0;
        }
    }
    p->n_qblk = (int)cdiv(sh.Sq, p->q_rows);
    // (head rows and head row groups: one workgroup per head_rows / fused_rg query heads)
    const int64_t heads_per_wg = p->fused_hg ? p->fused_rg : p->head_rows > 0 ? p->head_rows : 1;
    p->grid = sh.B * sh.Hq / heads_per_wg * p->n_qblk * (p->path == SDPA_PATH_FUSED ? p->n_splits : 1);
    p->tiles_per_bh = count_tiles(sh.Sq, sh.Skv, causal, p->q_rows, coff);
    if (p->grid > INT32_MAX) return fail(SDPA_ERR_UNSUPPORTED, "grid too large");
    return SDPA_OK;
}

// Strides (batch, head, row) in elements. A size-1 batch or head dim never
// advances (stride 0); a single row gets the row length as its pitch so that
// rows past the end fall outside the per-(batch, head) buffer descriptor.
void fill_strides3(const sdpa_tensor_t* t, int64_t* s) {
    for (int d = 0; d < 2; ++d) s[d] = eff_stride(t, d);
    s[2] = t->sizes[2] == 1 ? t->sizes[3] : t->strides[2];
}

// Where a call's key-range workspace comes from: the caller's buffer (NULL:
// none, run unsplit) or the library's per-device static scratch.
enum WsMode { WS_CALLER = 0, WS_STATIC = 1 };

// Dropout of one call: the caller's keep-mask, p and rule.
struct DropSpec {
    const sdpa_tensor_t* keep;
    float p;
    int rule;  // 0 explicit, 1 random
};

sdpa_status_t validate_dropout(const Shape& sh, const DropSpec& d) {
    if (!(d.p >= 0.0f && d.p < 1.0f)) return fail(SDPA_ERR_INVALID_ARG, "dropout_p must be in [0, 1), got %g", d.p);
    if (d.rule != 0 && d.rule != 1) return fail(SDPA_ERR_INVALID_ARG, "dropout rule must be 0 (explicit) or 1 (random)");
    const sdpa_tensor_t* m = d.keep;
    if (!m) return fail(SDPA_ERR_INVALID_ARG, "dropout needs a keep-mask");
    if (m->ndim != 4) return fail(SDPA_ERR_INVALID_ARG, "the keep-mask must be passed with 4 dims (right-aligned)");
    if (m->dtype != SDPA_BOOL) return fail(SDPA_ERR_INVALID_ARG, "the keep-mask must be bool");
    const int64_t full[4] = {sh.B, sh.Hq, sh.Sq, sh.Skv};
    for (int dd = 0; dd < 4; ++dd)
        if (m->sizes[dd] < 0 || (m->sizes[dd] != 1 && m->sizes[dd] != full[dd]))
            return fail(SDPA_ERR_INVALID_ARG, "keep-mask dim %d (%lld) does not broadcast to %lld", dd,
                        (long long)m->sizes[dd], (long long)full[dd]);
    if (numel(m) > 0 && !m->data) return fail(SDPA_ERR_INVALID_ARG, "the keep-mask has no data pointer");
    return SDPA_OK;
}

sdpa_status_t run(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v, const sdpa_tensor_t* mask,
                  int is_causal, float scale, int enable_gqa, sdpa_tensor_t* out, sdpa_tensor_t* probs,
                  sdpa_tensor_t* lse, void* stream, int path, void* ws = nullptr, size_t ws_bytes = 0,
                  WsMode ws_mode = WS_CALLER, const DropSpec* drop = nullptr) {
    g_last_error.clear();
    if (path < SDPA_PATH_AUTO || path > SDPA_PATH_TWOPASS) return fail(SDPA_ERR_INVALID_ARG, "unknown path %d", path);
    Shape sh;
    sdpa_status_t st = validate_inputs(q, k, v, mask, is_causal, enable_gqa, &sh);
    if (st) return st;
    if ((st = validate_outputs(sh, out, probs, lse))) return st;
    if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale must be finite");
    if (drop) {
        if ((st = validate_dropout(sh, *drop))) return st;
        // [FlagOS] single-kernel fusion update: dropout always takes the two-stage path
        if (path == SDPA_PATH_FUSED) return fail(SDPA_ERR_UNSUPPORTED, "dropout runs on the two-pass path only");
        path = SDPA_PATH_TWOPASS;
        ws = nullptr;
        ws_mode = WS_CALLER;
    }
    if (sh.B * sh.Hq * sh.Sq == 0) return SDPA_OK;
    const bool vec = staged_layout(sh, mask, out, probs);
    sdpa::Plan plan;
    if ((st = make_plan(sh, is_causal != 0, causal_offset(sh, is_causal), path, vec, &plan,
                        ws_mode == WS_STATIC || ws != nullptr)))
        return st;
    // the wide kernel's key ranges without room for their workspace: the
    // two-pass split instead (whose workspace is checked below)
    if (plan.path == SDPA_PATH_FUSED && plan.n_splits > 1) {
        const size_t room = ws_mode == WS_STATIC                           ? sdpa::STATIC_SCRATCH_BYTES
                            : reinterpret_cast<uintptr_t>(ws) % 256 != 0 ? 0
                                                                          : ws_bytes;
        if (plan_ws_bytes(sh, plan) > room &&
            (st = make_plan(sh, is_causal != 0, causal_offset(sh, is_causal), path, vec, &plan, true, false)))
            return st;
    }
    if (ws_mode == WS_STATIC && plan.n_splits > 1) {
        // the static scratch: a plan that needs more is rejected, never shrunk
        const size_t need = plan_ws_bytes(sh, plan);
        if (need > sdpa::STATIC_SCRATCH_BYTES)
            return fail(SDPA_ERR_UNSUPPORTED,
                        "this call needs %zu bytes of key-range scratch; the static scratch holds %zu "
                        "(use sdpa_math_fwd_ws with a caller workspace)",
                        need, sdpa::STATIC_SCRATCH_BYTES);
        const int e = sdpa::static_scratch(&ws);
        if (e != 0)
            return fail(SDPA_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(static_cast<hipError_t>(e)));
        ws_bytes = sdpa::STATIC_SCRATCH_BYTES;
    }
    if (plan.n_splits > 1 && (reinterpret_cast<uintptr_t>(ws) % 256 != 0 || ws_bytes < plan_ws_bytes(sh, plan)))
        if ((st = make_plan(sh, is_causal != 0, causal_offset(sh, is_causal), path, vec, &plan))) return st;  // no room: unsplit
    if (drop) {  // the dropout kernels: two compute waves and a loader wave
        plan.waves = 2;
        plan.q_rows = 64;
        plan.n_qblk = (int)cdiv(sh.Sq, 64);
        plan.grid = sh.B * sh.Hq * plan.n_qblk;
        plan.tiles_per_bh = count_tiles(sh.Sq, sh.Skv, is_causal != 0, 64, causal_offset(sh, is_causal));
    }

    sdpa::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.mask = mask ? mask->data : nullptr;
    a.o = out->data;
    a.p = probs->data;
    a.lse = static_cast<float*>(lse->data);
    fill_strides3(q, a.q_s);
    fill_strides3(k, a.k_s);
    fill_strides3(v, a.v_s);
    fill_strides3(out, a.o_s);
    fill_strides3(probs, a.p_s);
    for (int d = 0; d < 3; ++d) a.l_s[d] = eff_stride(lse, d);
    if (mask)
        for (int d = 0; d < 4; ++d) a.m_s[d] = eff_stride(mask, d);
    a.B = (int)sh.B;
    a.Hq = (int)sh.Hq;
    a.Hkv = (int)sh.Hkv;
    a.Sq = (int)sh.Sq;
    a.Skv = (int)sh.Skv;
    a.group = (int)(sh.Hq / sh.Hkv);
    a.causal = is_causal ? 1 : 0;
    a.coff = (int)causal_offset(sh, is_causal);
    const int64_t es = elt_size(sh.dtype);
    const int64_t me = sh.mask_kind == sdpa::MASK_BOOL ? 1 : es;
    a.mask_vec = vec && mask;
    a.p_vec = vec;
    a.o_vec = vec;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.n_qblk = plan.n_qblk;
    a.n_blocks = (int)plan.grid;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    if (plan.n_splits > 1) {
        a.ws_ml = static_cast<float2*>(ws);
        a.ws_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (split_ws_ml_bytes(sh, plan.n_splits) + 255) / 256 * 256);
        if (plan.path == SDPA_PATH_FUSED)
            a.ws_e = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + plan_ws_e_offset(sh, plan.n_splits));
    }
    a.keys_per_wave = plan.keys_per_wave;
    a.fused_rg = plan.fused_rg;
    a.fused_hg = plan.fused_hg;
    a.fused_oseq = plan.fused_oseq;
    a.head_rows = plan.head_rows;
    if (drop) {
        a.keep = static_cast<const uint8_t*>(drop->keep->data);
        for (int dd = 0; dd < 4; ++dd) a.kp_s[dd] = eff_stride(drop->keep, dd);
        const int64_t kext = sh.Skv > 0 ? (sh.Sq - 1) * a.kp_s[2] + (sh.Skv - 1) * a.kp_s[3] + 1 : 0;
        if (kext >= (int64_t(1) << 30)) return fail(SDPA_ERR_UNSUPPORTED, "one (batch, head) slice spans 1 GiB or more");
        a.kp_ext = (uint32_t)kext;
        a.keep_vec = a.kp_s[3] == 1 && sh.Skv % 8 == 0 && reinterpret_cast<uintptr_t>(a.keep) % 8 == 0 &&
                     (a.kp_s[0] % 8) == 0 && (a.kp_s[1] % 8) == 0 && (a.kp_s[2] % 8) == 0;
        a.drop_oscale = (float)(1.0 / (1.0 - (double)drop->p));
        a.drop_pscale = drop->rule == 1 ? a.drop_oscale : 1.0f;
    }
    // Workgroup order (decode_block). Non-causal: head-major, each XCD taking
    // consecutive blocks (shared K/V in its L2). Causal: when the grid is
    // more than one round of resident workgroups (two per CU on 256 CUs),
    // each XCD takes its heads two at a time, their blocks heaviest first
    // (needs an even number of whole heads per XCD): 2k x 2k D=128, 704
    // blocks, 91 us against 103 head-major and 110 grid-wide heaviest-first.
    // Otherwise heaviest first over the whole grid: 1k x 1k D=64, 352
    // blocks, all resident at once, 23.6 us against 26.7 with head pairs.
    // Head rows (non-causal): dispatch order (order 4), so that every XCD
    // takes a share of every batch: GQA key padding (per-batch key counts
    // 601 to 1017) 139.4 us against 157.0 with each XCD's heads advancing
    // together (order 5) and 151.4 with those heads strided over batches.
    // SDPA_MATH_SCHED=0..5 overrides (1: heavy and light blocks interleaved
    // per XCD).
    constexpr int64_t kResidentWorkgroups = 2 * 256;
    const int64_t per_xcd = plan.grid % 8 == 0 ? plan.grid / 8 : 0;
    const bool pairs_ok = is_causal && per_xcd > 0 && per_xcd % (2 * plan.n_qblk) == 0;
    a.sched = is_causal ? ((pairs_ok && plan.grid > kResidentWorkgroups) ? 3 : 2) : plan.head_rows > 0 ? 4 : 0;
    if (const char* e = std::getenv("SDPA_MATH_SCHED")) {
        a.sched = 0;
        // order 1 splits each XCD's range into a heavy and a light half of
        // whole heads' blocks: a permutation only with an even block count
        if (*e == '1' && is_causal && per_xcd > 0 && per_xcd % plan.n_qblk == 0 && plan.n_qblk % 2 == 0) a.sched = 1;
        if (*e == '2' && is_causal) a.sched = 2;
        if (*e == '3' && pairs_ok) a.sched = 3;
        if (*e == '4') a.sched = 4;
        if (*e == '5') a.sched = 5;
    }

    // byte extent of one (batch, head) slice of each tensor
    int64_t ext[7];
    ext[0] = ((sh.Sq - 1) * a.q_s[2] + sh.D) * es;
    ext[1] = sh.Skv > 0 ? ((sh.Skv - 1) * a.k_s[2] + sh.D) * es : 0;
    ext[2] = sh.Skv > 0 ? ((sh.Skv - 1) * a.v_s[2] + sh.Dv) * es : 0;
    ext[3] = ((sh.Sq - 1) * a.o_s[2] + sh.Dv) * es;
    ext[4] = ((sh.Sq - 1) * a.p_s[2] + sh.Skv) * es;
    ext[5] = (mask && sh.Skv > 0) ? ((sh.Sq - 1) * a.m_s[2] + (sh.Skv - 1) * a.m_s[3] + 1) * me : 0;
    ext[6] = ((sh.Sq - 1) * a.l_s[2] + 1) * 4;
    for (int i = 0; i < 7; ++i)
        if (ext[i] < 0 || ext[i] >= (int64_t(1) << 30))
            return fail(SDPA_ERR_UNSUPPORTED, "one (batch, head) slice spans 1 GiB or more");
    a.q_ext = (uint32_t)ext[0];
    a.k_ext = (uint32_t)ext[1];
    a.v_ext = (uint32_t)ext[2];
    a.o_ext = (uint32_t)ext[3];
    a.p_ext = (uint32_t)ext[4];
    a.m_ext = (uint32_t)ext[5];
    a.l_ext = (uint32_t)ext[6];

    const int D = (int)sh.D;
    int err;
    if (plan.path == SDPA_PATH_FUSED) {
        err = sdpa::launch_fused(sh.dtype, D, sh.mask_kind, plan.waves, vec, a, stream);
    } else if (sh.dtype == SDPA_BF16) {
        err = sdpa::launch_twopass_bf16(D, sh.mask_kind, plan.waves, vec, drop != nullptr, a, stream);
    } else if (sh.dtype == SDPA_F16) {
        err = sdpa::launch_twopass_f16(D, sh.mask_kind, plan.waves, vec, drop != nullptr, a, stream);
    } else {
        err = sdpa::launch_twopass_f32(D, sh.mask_kind, plan.waves, vec, drop != nullptr, a, stream);
    }
    if (err != 0)
        return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(err)));
    if (std::getenv("SDPA_MATH_DEBUG"))
        std::fprintf(stderr, "sdpa_math: path=%s waves=%d vec=%d sched=%d splits=%d grid=%lld tiles/bh=%lld tiles64/bh=%lld\n",
                     plan.path == SDPA_PATH_FUSED ? "fused" : "twopass", plan.waves, vec ? 1 : 0, a.sched,
                     plan.n_splits, (long long)plan.grid,
                     (long long)plan.tiles_per_bh, (long long)plan.tiles_64);
    return SDPA_OK;
}

// Byte extent of one (batch, head) slice: `rows` rows of `cols` elements at
// a row pitch of `pitch` elements (0 rows: 0).
int64_t slice_extent(int64_t rows, int64_t pitch, int64_t cols, int64_t es) {
    return rows > 0 && cols > 0 ? ((rows - 1) * pitch + cols) * es : 0;
}

// Query ranges of the combined key-side backward launch (causal calls):
// when its key blocks (64 keys, two waves each) give fewer than two waves
// per SIMD of the chip (2048 waves), each key block's (query head, 32-row
// tile) steps are split over up to 4 workgroups of at least 8 steps each,
// whose float32 partial dk and dv a reduce launch sums. Under a causal mask
// the early key blocks have the most steps, and the ranges shorten that
// longest chain: 1k causal fp16 D = 64 186.9 -> 172.6 us. Without one every
// key block has the same work and the ranges only add their partials' round
// trip (GQA key padding 1841 -> 1917 us), so they are not taken.
int bwd_kv_splits(const Shape& sh, bool causal) {
    const int64_t nk = sh.B * sh.Hkv * cdiv(sh.Skv, 64);
    if (!causal || nk <= 0 || nk * 2 >= 2048) return 1;
    const int64_t steps = (sh.Hq / sh.Hkv) * cdiv(sh.Sq, 32);
    const int64_t ns = std::min<int64_t>({cdiv(2048, nk * 2), 4, std::max<int64_t>(1, steps / 8)});
    return (int)ns;
}

// Backward workspace: the per-row sum D_i = sum_j P_ij dP_ij in float32,
// then (query ranges) the ranges' float32 partial dk and dv.
size_t bwd_dsum_bytes(const Shape& sh) { return ((size_t)(sh.B * sh.Hq * sh.Sq) * 4 + 255) / 256 * 256; }
size_t bwd_ws_bytes(const Shape& sh, bool causal) {
    const int ns = bwd_kv_splits(sh, causal);
    return bwd_dsum_bytes(sh) + (ns > 1 ? (size_t)ns * 2 * (size_t)(sh.B * sh.Hkv * sh.Skv * sh.D) * 4 : 0);
}

sdpa_status_t check_grad(const sdpa_tensor_t* t, const char* name, int dtype, const int64_t* want, int ndim,
                         bool aligned) {
    sdpa_status_t st;
    if ((st = check_tensor(t, name, ndim))) return st;
    if (t->dtype != dtype)
        return fail(SDPA_ERR_INVALID_ARG, "%s must have dtype %s, got %s", name, dtype_name(dtype), dtype_name(t->dtype));
    if ((st = check_dims(t, name, want, ndim))) return st;
    if (aligned && numel(t) > 0 && !rows_aligned(t, 16))
        return fail(SDPA_ERR_UNSUPPORTED, "%s needs a 16-byte aligned base and 16-byte multiple strides", name);
    return SDPA_OK;
}

sdpa_status_t run_bwd(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                      const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa, const sdpa_tensor_t* lse,
                      const sdpa_tensor_t* dout, const sdpa_tensor_t* dprobs, sdpa_tensor_t* dq, sdpa_tensor_t* dk,
                      sdpa_tensor_t* dv, void* ws, size_t ws_bytes, void* stream) {
    g_last_error.clear();
    Shape sh;
    sdpa_status_t st = validate_inputs(q, k, v, mask, is_causal, enable_gqa, &sh);
    if (st) return st;
    const int64_t wl[3] = {sh.B, sh.Hq, sh.Sq};
    const int64_t wo[4] = {sh.B, sh.Hq, sh.Sq, sh.Dv};
    const int64_t wp[4] = {sh.B, sh.Hq, sh.Sq, sh.Skv};
    const int64_t wq[4] = {sh.B, sh.Hq, sh.Sq, sh.D};
    const int64_t wk[4] = {sh.B, sh.Hkv, sh.Skv, sh.D};
    const int64_t wv[4] = {sh.B, sh.Hkv, sh.Skv, sh.Dv};
    if ((st = check_grad(lse, "lse", SDPA_F32, wl, 3, false)) || (st = check_grad(dout, "dout", sh.dtype, wo, 4, true)) ||
        (dprobs && (st = check_grad(dprobs, "dprobs", sh.dtype, wp, 4, false))) ||
        (st = check_grad(dq, "dq", sh.dtype, wq, 4, true)) || (st = check_grad(dk, "dk", sh.dtype, wk, 4, true)) ||
        (st = check_grad(dv, "dv", sh.dtype, wv, 4, true)))
        return st;
    if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale must be finite");
    if (sh.B * sh.Hkv == 0) return SDPA_OK;
    const size_t need = bwd_ws_bytes(sh, is_causal != 0);
    if (need > 0 && (!ws || reinterpret_cast<uintptr_t>(ws) % 16 != 0 || ws_bytes < need))
        return fail(SDPA_ERR_INVALID_ARG, "the backward needs a 16-byte aligned workspace of %zu bytes "
                                          "(sdpa_math_bwd_workspace_bytes)", need);

    sdpa::BwdArgs a;
    std::memset(&a, 0, sizeof a);
    sdpa::FwdArgs& f = a.f;
    f.q = q->data;
    f.k = k->data;
    f.v = v->data;
    f.mask = mask ? mask->data : nullptr;
    f.lse = static_cast<float*>(lse->data);
    fill_strides3(q, f.q_s);
    fill_strides3(k, f.k_s);
    fill_strides3(v, f.v_s);
    for (int d = 0; d < 3; ++d) f.l_s[d] = eff_stride(lse, d);
    if (mask)
        for (int d = 0; d < 4; ++d) f.m_s[d] = eff_stride(mask, d);
    f.B = (int)sh.B;
    f.Hq = (int)sh.Hq;
    f.Hkv = (int)sh.Hkv;
    f.Sq = (int)sh.Sq;
    f.Skv = (int)sh.Skv;
    f.group = (int)(sh.Hq / sh.Hkv);
    f.causal = is_causal ? 1 : 0;
    f.coff = (int)causal_offset(sh, is_causal);
    f.scale_log2 = scale * 1.4426950408889634f;
    a.scale = scale;
    a.dout = dout->data;
    a.dprobs = dprobs ? dprobs->data : nullptr;
    a.dq = dq->data;
    a.dk = dk->data;
    a.dv = dv->data;
    a.dsum = static_cast<float*>(ws);
    a.kv_splits = bwd_kv_splits(sh, is_causal != 0);
    if (a.kv_splits > 1) a.ws_kv = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + bwd_dsum_bytes(sh));
    fill_strides3(dout, a.do_s);
    if (dprobs) fill_strides3(dprobs, a.dp_s);
    fill_strides3(dq, a.dq_s);
    fill_strides3(dk, a.dk_s);
    fill_strides3(dv, a.dv_s);
    const int64_t es = elt_size(sh.dtype);
    const int64_t me = sh.mask_kind == sdpa::MASK_BOOL ? 1 : es;
    a.dp_vec = dprobs && rows_aligned(dprobs, 16) && sh.Skv % 8 == 0;
    f.mask_vec = mask && eff_stride(mask, 3) == 1 && rows_aligned(mask, 16) && sh.Skv % 8 == 0;
    int64_t ext[10];
    ext[0] = slice_extent(sh.Sq, f.q_s[2], sh.D, es);
    ext[1] = slice_extent(sh.Skv, f.k_s[2], sh.D, es);
    ext[2] = slice_extent(sh.Skv, f.v_s[2], sh.Dv, es);
    ext[3] = (mask && sh.Skv > 0 && sh.Sq > 0) ? ((sh.Sq - 1) * f.m_s[2] + (sh.Skv - 1) * f.m_s[3] + 1) * me : 0;
    ext[4] = slice_extent(sh.Sq, f.l_s[2], 1, 4);
    ext[5] = slice_extent(sh.Sq, a.do_s[2], sh.Dv, es);
    ext[6] = dprobs ? slice_extent(sh.Sq, a.dp_s[2], sh.Skv, es) : 0;
    ext[7] = slice_extent(sh.Sq, a.dq_s[2], sh.D, es);
    ext[8] = slice_extent(sh.Skv, a.dk_s[2], sh.D, es);
    ext[9] = slice_extent(sh.Skv, a.dv_s[2], sh.Dv, es);
    for (int i = 0; i < 10; ++i)
        if (ext[i] < 0 || ext[i] >= (int64_t(1) << 30))
            return fail(SDPA_ERR_UNSUPPORTED, "one (batch, head) slice spans 1 GiB or more");
    f.q_ext = (uint32_t)ext[0];
    f.k_ext = (uint32_t)ext[1];
    f.v_ext = (uint32_t)ext[2];
    f.m_ext = (uint32_t)ext[3];
    f.l_ext = (uint32_t)ext[4];
    a.do_ext = (uint32_t)ext[5];
    a.dp_ext = (uint32_t)ext[6];
    a.dq_ext = (uint32_t)ext[7];
    a.dk_ext = (uint32_t)ext[8];
    a.dv_ext = (uint32_t)ext[9];
    const int err = sdpa::launch_backward(sh.dtype, (int)sh.D, sh.mask_kind, a, stream);
    if (err != 0)
        return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(err)));
    return SDPA_OK;
}

// Packed variable-length sequences (THD): q [Tq, Hq, D], k [Tkv, Hkv, D],
// v [Tkv, Hkv, Dv], out [Tq, Hq, Dv], probs [Tq, Hq, max_skv], lse [Tq, Hq].
sdpa_status_t run_varlen(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v, const int32_t* cu_q,
                         const int32_t* cu_k, int64_t nseq, int64_t max_sq, int64_t max_skv, int is_causal, float scale,
                         int enable_gqa, sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* stream) {
    g_last_error.clear();
    sdpa_status_t st;
    if ((st = check_tensor(q, "q", 3)) || (st = check_tensor(k, "k", 3)) || (st = check_tensor(v, "v", 3)))
        return st;
    if (q->dtype != SDPA_F32 && q->dtype != SDPA_F16 && q->dtype != SDPA_BF16)
        return fail(SDPA_ERR_INVALID_ARG, "q dtype %s is not f32, f16 or bf16", dtype_name(q->dtype));
    if (k->dtype != q->dtype || v->dtype != q->dtype) return fail(SDPA_ERR_INVALID_ARG, "q, k, v dtypes differ");
    Shape sh;
    sh.B = nseq;
    sh.Hq = q->sizes[1];
    sh.D = q->sizes[2];
    sh.Hkv = k->sizes[1];
    sh.Dv = v->sizes[2];
    sh.Sq = max_sq;
    sh.Skv = max_skv;
    sh.dtype = q->dtype;
    sh.mask_kind = sdpa::MASK_NONE;
    sh.mask_head_shared = true;
    const int64_t Tq = q->sizes[0], Tkv = k->sizes[0];
    if (nseq < 0 || max_sq < 0 || max_skv < 0)
        return fail(SDPA_ERR_INVALID_ARG, "sequence count and maximum lengths must be non-negative");
    if (nseq > 0 && (!cu_q || !cu_k)) return fail(SDPA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_kv are required");
    if (v->sizes[0] != Tkv || v->sizes[1] != sh.Hkv) return fail(SDPA_ERR_INVALID_ARG, "k and v disagree on tokens or heads");
    if (k->sizes[2] != sh.D) return fail(SDPA_ERR_INVALID_ARG, "q and k head dims differ");
    if (sh.Hkv <= 0 || sh.Hq % sh.Hkv != 0)
        return fail(SDPA_ERR_INVALID_ARG, "query heads (%lld) are not a multiple of key/value heads (%lld)",
                    (long long)sh.Hq, (long long)sh.Hkv);
    if (sh.Hq != sh.Hkv && !enable_gqa) return fail(SDPA_ERR_INVALID_ARG, "Hq != Hkv needs enable_gqa");
    if (is_causal < 0 || is_causal > 2) return fail(SDPA_ERR_INVALID_ARG, "is_causal must be 0, 1 or 2");
    if (Tq > INT32_MAX || Tkv > INT32_MAX || max_sq > INT32_MAX || max_skv > INT32_MAX || nseq > INT32_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "sizes beyond 2^31 are not supported");
    if (sh.D != 32 && sh.D != 64 && sh.D != 128)
        return fail(SDPA_ERR_UNSUPPORTED, "head dim %lld is not implemented (32, 64, 128)", (long long)sh.D);
    if (sh.Dv != sh.D) return fail(SDPA_ERR_UNSUPPORTED, "value head dim != query head dim is not implemented");
    const sdpa_tensor_t* in[3] = {q, k, v};
    for (int i = 0; i < 3; ++i)
        if (numel(in[i]) > 0 && !rows_aligned(in[i], 16))
            return fail(SDPA_ERR_UNSUPPORTED, "q, k, v need 16-byte aligned bases and 16-byte multiple strides");
    const int64_t wo[3] = {Tq, sh.Hq, sh.Dv};
    const int64_t wp[3] = {Tq, sh.Hq, max_skv};
    if ((st = check_tensor(out, "out", 3)) || (st = check_tensor(probs, "probs", 3))) return st;
    if ((st = check_tensor(lse, "lse", 2))) return st;
    if (out->dtype != sh.dtype || probs->dtype != sh.dtype)
        return fail(SDPA_ERR_INVALID_ARG, "out and probs must have the query dtype");
    if (lse->dtype != SDPA_F32) return fail(SDPA_ERR_INVALID_ARG, "lse must be f32");
    const int64_t wl[2] = {Tq, sh.Hq};
    if ((st = check_dims(out, "out", wo, 3)) || (st = check_dims(probs, "probs", wp, 3)) ||
        (st = check_dims(lse, "lse", wl, 2)))
        return st;
    if (!std::isfinite(scale)) return fail(SDPA_ERR_INVALID_ARG, "scale must be finite");
    if (nseq == 0 || sh.Hq == 0 || max_sq == 0 || Tq == 0) return SDPA_OK;

    const int64_t es = elt_size(sh.dtype);
    const bool vec = max_skv % 8 == 0 && rows_aligned(out, 16) && rows_aligned(probs, 16);
    sdpa::FwdArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.o = out->data;
    a.p = probs->data;
    a.lse = static_cast<float*>(lse->data);
    // (batch, head, row) strides: no batch stride, tokens are the rows
    auto st3 = [](const sdpa_tensor_t* t, int64_t* s3) {
        s3[0] = 0;
        s3[1] = eff_stride(t, 1);
        s3[2] = t->strides[0];
    };
    st3(q, a.q_s);
    st3(k, a.k_s);
    st3(v, a.v_s);
    st3(out, a.o_s);
    st3(probs, a.p_s);
    a.l_s[0] = 0;
    a.l_s[1] = eff_stride(lse, 1);
    a.l_s[2] = lse->strides[0];
    a.B = (int)nseq;
    a.Hq = (int)sh.Hq;
    a.Hkv = (int)sh.Hkv;
    a.Sq = (int)max_sq;
    a.Skv = (int)max_skv;
    a.group = (int)(sh.Hq / sh.Hkv);
    a.causal = is_causal ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.p_vec = vec;
    a.o_vec = vec;
    a.n_qblk = (int)cdiv(max_sq, 64);
    const int64_t grid = nseq * sh.Hq * a.n_qblk;
    if (grid > INT32_MAX) return fail(SDPA_ERR_UNSUPPORTED, "grid too large");
    a.n_blocks = (int)grid;
    a.sched = 0;
    a.n_splits = 1;
    a.thd = 1;
    a.thd_bottom_right = is_causal == 2;
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.Tq = (int)Tq;
    a.Tkv = (int)Tkv;
    a.p_cols = (int)max_skv;
    int64_t ext[6];
    ext[0] = slice_extent(max_sq, a.q_s[2], sh.D, es);
    ext[1] = slice_extent(max_skv, a.k_s[2], sh.D, es);
    ext[2] = slice_extent(max_skv, a.v_s[2], sh.Dv, es);
    ext[3] = slice_extent(max_sq, a.o_s[2], sh.Dv, es);
    ext[4] = slice_extent(max_sq, a.p_s[2], max_skv, es);
    ext[5] = slice_extent(max_sq, a.l_s[2], 1, 4);
    for (int i = 0; i < 6; ++i)
        if (ext[i] < 0 || ext[i] >= (int64_t(1) << 30))
            return fail(SDPA_ERR_UNSUPPORTED, "one (sequence, head) slice spans 1 GiB or more");
    a.q_ext = (uint32_t)ext[0];
    a.k_ext = (uint32_t)ext[1];
    a.v_ext = (uint32_t)ext[2];
    a.o_ext = (uint32_t)ext[3];
    a.p_ext = (uint32_t)ext[4];
    a.l_ext = (uint32_t)ext[5];
    const int D = (int)sh.D;
    int err;
    if (sh.dtype == SDPA_BF16) err = sdpa::launch_twopass_bf16(D, sdpa::MASK_NONE, 2, vec, false, a, stream);
    else if (sh.dtype == SDPA_F16) err = sdpa::launch_twopass_f16(D, sdpa::MASK_NONE, 2, vec, false, a, stream);
    else err = sdpa::launch_twopass_f32(D, sdpa::MASK_NONE, 2, vec, false, a, stream);
    if (err != 0)
        return fail(SDPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(err)));
    return SDPA_OK;
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_math_fwd(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                            const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                            sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* hip_stream) {
    return run(q, k, v, mask, is_causal, scale, enable_gqa, out, probs, lse, hip_stream, SDPA_PATH_AUTO);
}

sdpa_status_t sdpa_math_fwd_path(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                 const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                                 sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* hip_stream,
                                 int path) {
    return run(q, k, v, mask, is_causal, scale, enable_gqa, out, probs, lse, hip_stream, path);
}

sdpa_status_t sdpa_math_plan(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                             const sdpa_tensor_t* mask, int is_causal, int enable_gqa, int32_t* path,
                             int64_t* tiles_per_bh, int64_t* tiles_64) {
    g_last_error.clear();
    Shape sh;
    sdpa_status_t st = validate_inputs(q, k, v, mask, is_causal, enable_gqa, &sh);
    if (st) return st;
    sdpa::Plan plan;
    // as a call with its workspace (sdpa_math_fwd_ws) runs it
    if ((st = make_plan(sh, is_causal != 0, causal_offset(sh, is_causal), SDPA_PATH_AUTO,
                        staged_layout(sh, mask, nullptr, nullptr), &plan, true)))
        return st;
    if (path) *path = plan.path == SDPA_PATH_FUSED && plan.fused_rg > 0 ? SDPA_PATH_FUSED_WIDE : plan.path;
    if (tiles_per_bh) *tiles_per_bh = plan.tiles_per_bh;
    if (tiles_64) *tiles_64 = plan.tiles_64;
    return SDPA_OK;
}

sdpa_status_t sdpa_math_fwd_ws(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                               const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                               sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* workspace,
                               size_t workspace_bytes, void* hip_stream, int path) {
    return run(q, k, v, mask, is_causal, scale, enable_gqa, out, probs, lse, hip_stream, path, workspace,
               workspace_bytes);
}

sdpa_status_t sdpa_math_fwd_dropout(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                    const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                                    float dropout_p, const sdpa_tensor_t* keep, int rule, sdpa_tensor_t* out,
                                    sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* hip_stream) {
    const DropSpec d{keep, dropout_p, rule};
    return run(q, k, v, mask, is_causal, scale, enable_gqa, out, probs, lse, hip_stream, SDPA_PATH_AUTO, nullptr, 0,
               WS_CALLER, &d);
}

sdpa_status_t sdpa_math_fwd_varlen(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int64_t n_seqs,
                                   int64_t max_seqlen_q, int64_t max_seqlen_kv, int is_causal, float scale,
                                   int enable_gqa, sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse,
                                   void* hip_stream) {
    return run_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, n_seqs, max_seqlen_q, max_seqlen_kv, is_causal, scale,
                      enable_gqa, out, probs, lse, hip_stream);
}

sdpa_status_t sdpa_math_fwd_noalloc(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                    const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                                    sdpa_tensor_t* out, sdpa_tensor_t* probs, sdpa_tensor_t* lse, void* hip_stream,
                                    int path) {
    return run(q, k, v, mask, is_causal, scale, enable_gqa, out, probs, lse, hip_stream, path, nullptr, 0, WS_STATIC);
}

sdpa_status_t sdpa_math_workspace_bytes(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                        const sdpa_tensor_t* mask, int is_causal, int enable_gqa, size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(SDPA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    Shape sh;
    sdpa_status_t st = validate_inputs(q, k, v, mask, is_causal, enable_gqa, &sh);
    if (st) return st;
    if (sh.B * sh.Hq * sh.Sq == 0) return SDPA_OK;
    sdpa::Plan plan;
    if ((st = make_plan(sh, is_causal != 0, causal_offset(sh, is_causal), SDPA_PATH_AUTO,
                        staged_layout(sh, mask, nullptr, nullptr), &plan, true)))
        return st;
    *bytes = plan_ws_bytes(sh, plan);
    return SDPA_OK;
}

sdpa_status_t sdpa_math_bwd_workspace_bytes(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                                            const sdpa_tensor_t* mask, int is_causal, int enable_gqa, size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(SDPA_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    Shape sh;
    sdpa_status_t st = validate_inputs(q, k, v, mask, is_causal, enable_gqa, &sh);
    if (st) return st;
    *bytes = bwd_ws_bytes(sh, is_causal != 0);
    return SDPA_OK;
}

sdpa_status_t sdpa_math_bwd(const sdpa_tensor_t* q, const sdpa_tensor_t* k, const sdpa_tensor_t* v,
                            const sdpa_tensor_t* mask, int is_causal, float scale, int enable_gqa,
                            const sdpa_tensor_t* lse, const sdpa_tensor_t* dout, const sdpa_tensor_t* dprobs,
                            sdpa_tensor_t* dq, sdpa_tensor_t* dk, sdpa_tensor_t* dv, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
    return run_bwd(q, k, v, mask, is_causal, scale, enable_gqa, lse, dout, dprobs, dq, dk, dv, workspace,
                   workspace_bytes, hip_stream);
}

const char* sdpa_math_last_error(void) { return g_last_error.c_str(); }

int sdpa_math_version(void) { return SDPA_MATH_VERSION; }

}  // extern "C"
