// C ABI of libpagedkv.so: host-side argument checks, split choice, launches.
// Nothing here allocates, synchronises or reads device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "internal.h"

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace pkv {
void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
}
void clear_error() { g_last_error[0] = '\0'; }
}  // namespace pkv

namespace {

pkv_status fail(pkv_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

pkv_status ok() {
    pkv::clear_error();
    return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return PKV_OK;
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int32_t kMaxSplits = 256;
constexpr int32_t kMaxUnits = 65535;
constexpr int32_t kVecMaxGroup = 8;

int32_t elem_bytes(pkv_dtype d) { return d == PKV_BF16 ? 2 : 4; }

bool dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }

// Shared checks on the head geometry.
pkv_status check_heads(int32_t q_heads, int32_t kv_heads, int32_t head_dim, pkv_dtype dtype) {
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "unknown dtype %d", (int)dtype);
    if (q_heads <= 0 || kv_heads <= 0) return fail(PKV_EINVAL, "q_heads and kv_heads must be > 0");
    if (q_heads % kv_heads != 0)
        return fail(PKV_EINVAL, "q_heads (%d) is not a multiple of kv_heads (%d)", q_heads, kv_heads);
    if (head_dim <= 0 || head_dim % 8 != 0 || head_dim > 256)
        return fail(PKV_EINVAL, "head_dim %d: must be a positive multiple of 8, at most 256", head_dim);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(PKV_EUNSUPPORTED, "head_dim %d has no compiled kernel (64, 128, 256)", head_dim);
    return PKV_OK;
}

int32_t clamp_splits(int64_t s, int64_t cap) {
    if (s > cap) s = cap;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)(s < 1 ? 1 : s);
}

// Compute units of the current device (256 on MI355X if the query fails).
int32_t device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// Vector path.  Several units: about one dispatch round of work groups (two
// per CU), and at least 4 splits per unit so that the balanced deal can even
// out unequal lengths; at least 8 blocks (two per wave) per split.  Each work
// group pays a fixed cost (the deal, the start of its stream, the split-K
// hand-off) of several microseconds under a full stream, so more rounds of
// smaller pieces lose: 2 sequences of 16K/4K keys (D 128) 31 us at 16 splits
// against 63 us at 128; 4 of 32K/64K 145 us at 16 against 167 us at 64; 16
// of up to 8K (D 256) 96-101 us at 2-4 against 156 us at 16; 64 of up to
// 8K (D 128) 197-200 us at 2-4 splits, 215 us at 8.  One unit: one work group per CU -- a single short round in which
// every split's work group is on the critical path, each wave with the same
// number of blocks where the length allows (the 4096-key, 8-head decode step
// measured 434 us at 32 splits, 448 us at 24, 456 us at 28, 504 us at 36) --
// and at least 4 blocks (one per wave) per split: the 42-layer step at 1024
// keys measured 336 us at 16 splits against 362 us at 8, at 2048 keys 369 us
// at 32 against 383 us at 16.
int32_t pick_splits(int32_t units, int32_t kv_heads, int32_t keys, int32_t num_splits) {
    if (num_splits > 0) return num_splits < kMaxSplits ? num_splits : kMaxSplits;
    const int64_t base = (int64_t)(units > 0 ? units : 1) * kv_heads;
    const int64_t blocks = ((int64_t)(keys > 0 ? keys : 1) + 15) / 16;
    const int64_t per = units <= 1 ? 4 : 8;         // blocks per split at least
    if (units <= 1)
        return clamp_splits(((int64_t)device_cus() + base - 1) / base, blocks / per > 0 ? blocks / per : 1);
    const int64_t s = (2 * (int64_t)device_cus() + base / 2) / base;
    return clamp_splits(s > 4 ? s : 4, blocks / per > 0 ? blocks / per : 1);
}

// Plan of one attention call: which paths run, their split counts and the
// workspace layout (vector tickets | mfma tickets | vector partials | mfma
// partials).  The arrival counters come first, so their places depend on the
// units, kv heads and row tiles only, not on the split counts.
struct Plan {
    bool vec, mfma;
    int32_t splits;          // vector path
    int32_t gt;              // vector path rows per work group
    int32_t tiles, msplits;  // matrix-core path
    int32_t bm;
    size_t vec_ticket, vec_bytes, mfma_ticket, mfma_bytes;
    size_t ws_bytes;
};

Plan make_plan(int32_t units, int32_t max_seqlen_q, int32_t keys, int32_t q_heads, int32_t kv_heads,
               int32_t head_dim, int32_t num_splits, bool mfma_ok) {
    Plan pl{};
    const int32_t group = q_heads / kv_heads;
    const int32_t U = units > 0 ? units : 1;
    // A call whose units may have several query rows runs every unit on the
    // matrix cores, single-row ones included, in one launch: which units have
    // one row only the device knows, and a separate vector launch would run
    // after, not beside, the matrix-core one.
    // Single-row units with a GQA group of 8 also run on the matrix cores
    // where they can (bf16): the vector kernel holds one wave per SIMD there
    // (377 VGPRs at head_dim 256), while the matrix-core kernel streams the
    // chunks through LDS with eight rows of a 16-row tile live.  Same inputs,
    // same box: 4 sequences of 32K/64K keys, D 256, 333 against 389-515 us;
    // D 128, 195 against 295 us; 16 sequences of up to 8K, D 128, 64 against
    // 152 us; 64 sequences of up to 8K, D 256, 563 against 595 us.  Groups of
    // 4 and below stay on the vector kernel (D 128, 64 sequences: 198 against
    // 325 us).
    const bool g8_mfma = mfma_ok && group >= kVecMaxGroup;
    pl.vec = group <= kVecMaxGroup && max_seqlen_q <= 1 && !g8_mfma;
    pl.mfma = max_seqlen_q > 1 || group > kVecMaxGroup || g8_mfma;
    pl.splits = pick_splits(units, kv_heads, keys, num_splits);
    pl.gt = pkv::vec_group_rows(group);
    if (pl.vec && pl.splits > 1) {
        pl.vec_ticket = pkv::ticket_bytes(U, kv_heads);
        pl.vec_bytes = (size_t)pkv::vec_slots(U, pl.splits) * kv_heads * pl.gt * ((size_t)head_dim + 2) *
                       sizeof(float);
    }
    if (pl.mfma) {
        const int64_t rows = (int64_t)max_seqlen_q * group;
        pl.bm = pkv::mfma_rows_per_group(head_dim, rows);
        pl.tiles = (int32_t)((rows + pl.bm - 1) / pl.bm);
        const int64_t base = (int64_t)U * kv_heads * pl.tiles;
        const int64_t chunks = ((int64_t)(keys > 0 ? keys : 1) + pkv::mfma_chunk_keys(head_dim, rows) - 1) /
                               pkv::mfma_chunk_keys(head_dim, rows);
        // Library choice: about one round of work groups on the device (the
        // dealt splits are equal in size, and every split adds a BM x D partial
        // to merge), at least 8 chunks per split.
        const int64_t round = (int64_t)device_cus() * pkv::mfma_groups_per_cu(head_dim, rows);
        pl.msplits = num_splits > 0 ? clamp_splits(num_splits, chunks)
                                    : clamp_splits((round + base / 2) / base, chunks / 8 > 0 ? chunks / 8 : 1);
        if (pl.msplits > 1) {
            pl.mfma_ticket = pkv::ticket_bytes(U * pl.tiles, kv_heads);
            pl.mfma_bytes = (size_t)base * pl.msplits * pl.bm * ((size_t)head_dim + 2) * sizeof(float);
        }
    } else {
        pl.tiles = 0;
        pl.msplits = 1;
    }
    pl.ws_bytes = pl.vec_ticket + pl.mfma_ticket + pl.vec_bytes + pl.mfma_bytes;
    return pl;
}

// Bytes at the start of the workspace that hold arrival counters.
size_t plan_ticket_bytes(const Plan& pl) { return pl.vec_ticket + pl.mfma_ticket; }

// Row mode (fp32 calls with several query rows per unit): the vector path
// takes every row of every unit as its own single-query item, units *
// max_seqlen_q items in all.
int64_t row_items(int32_t units, int32_t max_seqlen_q) {
    return (int64_t)(units > 0 ? units : 1) * (max_seqlen_q > 0 ? max_seqlen_q : 1);
}
constexpr int64_t kMaxGridY = 65535;

// Enqueue the attention kernels for a fully checked parameter block.
pkv_status run_attention(pkv::AttnParams& p, pkv_dtype dtype, int32_t head_dim, const Plan& pl,
                         void* workspace, hipStream_t stream) {
    char* ws = (char*)workspace;
    p.num_splits = pl.splits;
    p.ws_ticket = nullptr;
    p.ws_o = p.ws_ml = nullptr;
    p.vec_units = p.row_mode ? (int32_t)row_items(p.num_units, p.max_seqlen_q) : p.num_units;
    p.vec_wgs = pkv::vec_slots(p.vec_units, pl.splits);
    if (pl.vec && p.num_units > 0 && p.vec_wgs > kMaxGridY)
        return fail(PKV_EUNSUPPORTED, "%d vector-path work groups per kv head exceed the grid limit: pass a "
                    "smaller num_splits", p.vec_wgs);
    if (pl.mfma && p.num_units > 0 &&
        (int64_t)pl.tiles * pl.msplits * (pl.msplits > 1 ? p.num_units : 1) >
            kMaxGridY)
        return fail(PKV_EUNSUPPORTED, "too many matrix-core work groups per kv head: pass a smaller num_splits");
    char* partials = ws + plan_ticket_bytes(pl);
    if (pl.vec_bytes) {
        const size_t n = (size_t)p.vec_wgs * p.kv_heads * pl.gt;
        p.ws_ticket = (int32_t*)ws;
        p.ws_o = (float*)partials;
        p.ws_ml = p.ws_o + n * head_dim;
    }
    p.mfma_tiles = pl.tiles;
    p.mfma_splits = pl.msplits;
    p.mfma_single = pl.mfma && !pl.vec;
    p.mws_ticket = nullptr;
    p.mws_o = p.mws_ml = nullptr;
    if (pl.mfma_bytes) {
        const size_t n = (size_t)p.num_units * p.kv_heads * pl.tiles * pl.msplits * pl.bm;
        p.mws_ticket = (int32_t*)(ws + pl.vec_ticket);
        p.mws_o = (float*)(partials + pl.vec_bytes);
        p.mws_ml = p.mws_o + n * head_dim;
    }
    if (p.num_units == 0 && p.total_q == 0) return ok();
    // Rows no unit covers are zeroed inside the attention launch (the
    // matrix-core one when there is one), or by a launch of their own when
    // there is no unit to attend.
    p.zero_rows = (p.mode != pkv::kPagedDecode && p.num_units > 0) ? 1 : 0;
    if (p.mode != pkv::kPagedDecode && p.num_units == 0) {
        pkv_status s = hip_status(pkv::launch_zero_uncovered(p, dtype, head_dim, stream), "zero rows");
        if (s != PKV_OK) return s;
    }
    if (p.num_units > 0 && pl.vec) {
        pkv::AttnParams pv = p;
        pv.zero_rows = pl.mfma ? 0 : p.zero_rows;
        pkv_status s = hip_status(pkv::launch_attn_vec(pv, dtype, head_dim, stream), "attention");
        if (s != PKV_OK) return s;
    }
    if (p.num_units > 0 && pl.mfma) {
        pkv_status s = hip_status(pkv::launch_attn_mfma(p, dtype, head_dim, stream), "attention (mfma)");
        if (s != PKV_OK) return s;
    }
    return ok();
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_EINVAL: return "invalid argument";
        case PKV_EUNSUPPORTED: return "unsupported configuration";
        case PKV_EWORKSPACE: return "workspace too small";
        case PKV_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error; }

pkv_status pkv_kv_append(void* k_cache, void* v_cache, int64_t num_slots, const void* k_new,
                         const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                         int32_t kv_heads, int32_t head_dim, pkv_dtype dtype, void* stream) {
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "unknown dtype %d", (int)dtype);
    if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens must be >= 0");
    if (kv_heads <= 0 || head_dim <= 0 || head_dim % 8 != 0)
        return fail(PKV_EINVAL, "kv_heads must be > 0 and head_dim a positive multiple of 8");
    if (num_slots <= 0) return fail(PKV_EINVAL, "num_slots must be > 0");
    if (num_tokens == 0) return ok();
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
        return fail(PKV_EINVAL, "null pointer argument");
    const int64_t row_bytes = (int64_t)kv_heads * head_dim * elem_bytes(dtype);
    return hip_status(pkv::launch_kv_append(k_cache, v_cache, num_slots, k_new, v_new, num_tokens,
                                            slot_mapping, row_bytes, (hipStream_t)stream),
                      "kv_append");
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Shared checks of the two prefix copies; fills row_bytes on success.
pkv_status check_prefix(int32_t num_blocks, int32_t block_size, int32_t batch, int32_t n,
                        int32_t max_blocks_per_seq, int32_t kv_heads, int32_t head_dim,
                        pkv_dtype dtype, int64_t* row_bytes) {
    if (!dtype_ok(dtype)) return fail(PKV_EINVAL, "unknown dtype %d", (int)dtype);
    if (block_size != PKV_BLOCK_SIZE) return fail(PKV_EINVAL, "block_size %d: must be 16", block_size);
    if (kv_heads <= 0 || head_dim <= 0 || head_dim % 8 != 0)
        return fail(PKV_EINVAL, "kv_heads must be > 0 and head_dim a positive multiple of 8");
    if (num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_EINVAL, "num_blocks and max_blocks_per_seq must be > 0");
    if (batch < 0 || n < 0) return fail(PKV_EINVAL, "batch and n must be >= 0");
    if ((int64_t)n > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
        return fail(PKV_EINVAL, "n = %d exceeds 16 * max_blocks_per_seq", n);
    *row_bytes = (int64_t)head_dim * elem_bytes(dtype);
    // One work group per (sequence, block of 16 positions); 32-bit chunk index.
    if ((int64_t)batch * ((n + 15) / 16) >= ((int64_t)1 << 24) ||
        (int64_t)16 * kv_heads * (*row_bytes / 16) >= ((int64_t)1 << 30))
        return fail(PKV_EINVAL, "prefix copy too large for one launch");
    return PKV_OK;
}

}  // namespace

pkv_status pkv_prefix_import(void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size,
                             const void* k_src, const void* v_src, int32_t batch, int32_t src_len,
                             int32_t n, const int32_t* block_table, int32_t max_blocks_per_seq,
                             int32_t* seqused_k, int32_t kv_heads, int32_t head_dim,
                             pkv_dtype dtype, void* stream) {
    int64_t row_bytes = 0;
    pkv_status s = check_prefix(num_blocks, block_size, batch, n, max_blocks_per_seq, kv_heads,
                                head_dim, dtype, &row_bytes);
    if (s != PKV_OK) return s;
    if (src_len < n) return fail(PKV_EINVAL, "src_len %d < n %d", src_len, n);
    if (batch == 0 || (n == 0 && !seqused_k)) return ok();
    if (n > 0 && (!k_cache || !v_cache || !k_src || !v_src || !block_table))
        return fail(PKV_EINVAL, "null pointer argument");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_src) || !aligned16(v_src))
        return fail(PKV_EINVAL, "cache and source pointers must be 16-byte aligned");
    return hip_status(pkv::launch_prefix_copy(false, k_cache, v_cache, k_src, v_src, block_table,
                                              max_blocks_per_seq, num_blocks, batch, n, src_len,
                                              kv_heads, row_bytes, seqused_k, (hipStream_t)stream),
                      "prefix_import");
}

pkv_status pkv_prefix_export(void* k_dst, void* v_dst, const void* k_cache, const void* v_cache,
                             int32_t num_blocks, int32_t block_size, int32_t batch, int32_t n,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             int32_t kv_heads, int32_t head_dim, pkv_dtype dtype, void* stream) {
    int64_t row_bytes = 0;
    pkv_status s = check_prefix(num_blocks, block_size, batch, n, max_blocks_per_seq, kv_heads,
                                head_dim, dtype, &row_bytes);
    if (s != PKV_OK) return s;
    if (batch == 0 || n == 0) return ok();
    if (!k_dst || !v_dst || !k_cache || !v_cache || !block_table)
        return fail(PKV_EINVAL, "null pointer argument");
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_dst) || !aligned16(v_dst))
        return fail(PKV_EINVAL, "cache and destination pointers must be 16-byte aligned");
    return hip_status(pkv::launch_prefix_copy(true, k_dst, v_dst, k_cache, v_cache, block_table,
                                              max_blocks_per_seq, num_blocks, batch, n, n,
                                              kv_heads, row_bytes, nullptr, (hipStream_t)stream),
                      "prefix_export");
}

size_t pkv_attn_workspace_bytes(int32_t units, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                int32_t num_splits) {
    if (units <= 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || head_dim <= 0) return 0;
    // The plan depends on the dtype (bf16 may take the matrix cores, fp32 the
    // vector path, row by row for several rows per unit): cover every plan.
    size_t need = make_plan(units, max_seqlen_q, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits, true).ws_bytes;
    const size_t vec_need =
        make_plan(units, max_seqlen_q, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits, false).ws_bytes;
    if (vec_need > need) need = vec_need;
    const int64_t items = row_items(units, max_seqlen_q);
    if (max_seqlen_q > 1 && q_heads / kv_heads <= kVecMaxGroup && items <= INT32_MAX) {
        const size_t rows =
            make_plan((int32_t)items, 1, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits, false).ws_bytes;
        if (rows > need) need = rows;
    }
    return need;
}

int32_t pkv_attn_num_splits(int32_t units, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                            int32_t num_splits) {
    if (kv_heads <= 0) return 1;
    // As a bf16 call would split (head_dim 64/128/256).
    const Plan pl = make_plan(units, max_seqlen_q, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits, true);
    return pl.vec ? pl.splits : pl.msplits;
}

}  // extern "C"

namespace pkv {

pkv_status decode_check(void* out, const void* q, const void* k_cache, const void* v_cache,
                        int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seqused_k, int32_t num_seqs,
                        int32_t max_seqlen_k, const void* k_new, const void* v_new,
                        int32_t q_heads, int32_t kv_heads, int32_t head_dim, float softmax_scale,
                        int32_t num_splits, pkv_dtype dtype, size_t* ws_bytes, size_t* ticket_bytes) {
    *ws_bytes = 0;
    *ticket_bytes = 0;
    pkv_status s = check_heads(q_heads, kv_heads, head_dim, dtype);
    if (s != PKV_OK) return s;
    if (block_size != PKV_BLOCK_SIZE) return fail(PKV_EINVAL, "block_size %d: must be 16", block_size);
    if (num_seqs < 0 || num_seqs > kMaxUnits) return fail(PKV_EINVAL, "num_seqs out of range");
    if (num_blocks <= 0 || max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "num_blocks and max_blocks_per_seq must be > 0");
    if (max_seqlen_k < 0) return fail(PKV_EINVAL, "max_seqlen_k must be >= 0");
    if (num_splits < 0) return fail(PKV_EINVAL, "num_splits must be >= 0");
    if ((k_new == nullptr) != (v_new == nullptr)) return fail(PKV_EINVAL, "give both k_new and v_new, or neither");
    if (!isfinite(softmax_scale)) return fail(PKV_EINVAL, "softmax_scale must be finite");
    const int32_t group = q_heads / kv_heads;
    if (group > kVecMaxGroup && !pkv::attn_mfma_supported(dtype, head_dim))
        return fail(PKV_EUNSUPPORTED, "q_heads / kv_heads = %d > 8 needs bf16 (matrix-core path)", group);
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_table || !seqused_k)
        return fail(PKV_EINVAL, "null pointer argument");
    const Plan pl = make_plan(num_seqs, 1, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits,
                              pkv::attn_mfma_supported(dtype, head_dim));
    *ws_bytes = pl.ws_bytes;
    *ticket_bytes = plan_ticket_bytes(pl);
    return PKV_OK;
}

}  // namespace pkv

extern "C" {

pkv_status pkv_paged_decode_attn(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seqused_k,
                                 int32_t num_seqs, int32_t max_seqlen_k, const void* k_new,
                                 const void* v_new, int32_t q_heads, int32_t kv_heads,
                                 int32_t head_dim, float softmax_scale, int32_t causal,
                                 int32_t window, const int32_t* kv_start, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                                 void* stream) {
    size_t need = 0, tickets = 0;
    pkv_status s = pkv::decode_check(out, q, k_cache, v_cache, num_blocks, block_size, block_table,
                                     max_blocks_per_seq, seqused_k, num_seqs, max_seqlen_k, k_new, v_new,
                                     q_heads, kv_heads, head_dim, softmax_scale, num_splits, dtype, &need,
                                     &tickets);
    if (s != PKV_OK) return s;
    if (num_seqs == 0) return ok();
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(PKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const Plan pl = make_plan(num_seqs, 1, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits,
                              pkv::attn_mfma_supported(dtype, head_dim));
    const int32_t group = q_heads / kv_heads;

    const int64_t cap64 = (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE;
    const int32_t kv_cap = (int32_t)(cap64 < max_seqlen_k ? cap64 : max_seqlen_k);
    hipStream_t st = (hipStream_t)stream;
    pkv::AttnParams p{};
    // The vector kernel appends inside the attention; on the matrix-core path
    // (bf16 groups of 8 and above) the append goes first as its own launch.
    const bool append_first = k_new && !pl.vec;
    if (append_first) {
        pkv_status s2 = hip_status(
            pkv::launch_decode_append(const_cast<void*>(k_cache), const_cast<void*>(v_cache), num_blocks, k_new,
                                      v_new, num_seqs, (int64_t)kv_heads * head_dim * elem_bytes(dtype),
                                      seqused_k, kv_cap, block_table, max_blocks_per_seq, st),
            "decode append");
        if (s2 != PKV_OK) return s2;
    }
    p.k_new = append_first ? nullptr : k_new;
    p.v_new = append_first ? nullptr : v_new;
    p.out = out;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.seqused_k = seqused_k;
    p.block_table = block_table;
    p.kv_start = kv_start;
    p.mode = pkv::kPagedDecode;
    p.total_q = num_seqs;
    p.num_units = num_seqs;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.max_seqlen_q = 1;
    p.kv_cap = kv_cap;
    p.q_heads = q_heads;
    p.kv_heads = kv_heads;
    p.group = group;
    p.causal = causal != 0;
    p.window = window > 0 ? window : 0;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    return run_attention(p, dtype, head_dim, pl, workspace, st);
}

pkv_status pkv_varlen_attn(void* out, const void* q, int32_t total_q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_k, int32_t num_seqs,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t block_size, const int32_t* seq_info,
                           int32_t num_segments, int32_t rows, int32_t cols, int32_t max_seqlen_q,
                           int32_t max_seqlen_k, int32_t q_heads, int32_t kv_heads,
                           int32_t head_dim, float softmax_scale, int32_t causal, int32_t window,
                           const int32_t* kv_start, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, pkv_dtype dtype, void* stream) {
    pkv_status s = check_heads(q_heads, kv_heads, head_dim, dtype);
    if (s != PKV_OK) return s;
    const bool paged = block_table != nullptr;
    const bool column = seq_info != nullptr;
    if (paged == column) return fail(PKV_EINVAL, "give exactly one of block_table and seq_info");
    if (total_q < 0) return fail(PKV_EINVAL, "total_q must be >= 0");
    if (max_seqlen_q < 1) return fail(PKV_EINVAL, "max_seqlen_q must be >= 1");
    if (num_splits < 0) return fail(PKV_EINVAL, "num_splits must be >= 0");
    if (!isfinite(softmax_scale)) return fail(PKV_EINVAL, "softmax_scale must be finite");
    const int32_t w = window > 0 ? window : 0;
    int32_t units;
    if (paged) {
        if (block_size != PKV_BLOCK_SIZE) return fail(PKV_EINVAL, "block_size %d: must be 16", block_size);
        if (num_seqs < 0 || num_seqs > kMaxUnits) return fail(PKV_EINVAL, "num_seqs out of range");
        if (num_blocks <= 0 || max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "num_blocks and max_blocks_per_seq must be > 0");
        if (max_seqlen_k < 0) return fail(PKV_EINVAL, "max_seqlen_k must be >= 0");
        if (num_seqs > 0 && (!cu_seqlens_q || !seqused_k)) return fail(PKV_EINVAL, "null pointer argument");
        units = num_seqs;
    } else {
        if (rows <= 0 || cols <= 0) return fail(PKV_EINVAL, "rows and cols must be > 0");
        if (num_segments < 0) return fail(PKV_EINVAL, "num_segments must be >= 0");
        if ((int64_t)num_segments > 2 * (int64_t)cols)
            return fail(PKV_EINVAL, "num_segments %d > 2 * cols (%d)", num_segments, 2 * cols);
        if (w > 0 && (int64_t)rows < (int64_t)w + max_seqlen_q - 1)
            return fail(PKV_EINVAL, "ring of %d rows cannot hold window %d + max_seqlen_q %d - 1",
                        rows, w, max_seqlen_q);
        if (max_seqlen_k <= 0) return fail(PKV_EINVAL, "max_seqlen_k must be > 0 (bound on keys a segment sees)");
        units = num_segments;
    }
    const int32_t group = q_heads / kv_heads;
    if (group > kVecMaxGroup && !pkv::attn_mfma_supported(dtype, head_dim))
        return fail(PKV_EUNSUPPORTED, "q_heads / kv_heads = %d > 8 runs on the bf16 matrix-core path only", group);
    // fp32 with several rows per unit: every row on the vector path (row mode).
    const bool row_mode = max_seqlen_q > 1 && !pkv::attn_mfma_supported(dtype, head_dim);
    if (row_mode && row_items(units, max_seqlen_q) > INT32_MAX)
        return fail(PKV_EUNSUPPORTED, "units * max_seqlen_q too large for the fp32 row path");
    if (total_q == 0) return ok();
    if (!out || !q || !k || !v) return fail(PKV_EINVAL, "null pointer argument");
    const Plan pl = row_mode ? make_plan((int32_t)row_items(units, max_seqlen_q), 1, max_seqlen_k, q_heads, kv_heads,
                                         head_dim, num_splits, false)
                             : make_plan(units, max_seqlen_q, max_seqlen_k, q_heads, kv_heads, head_dim, num_splits,
                                         pkv::attn_mfma_supported(dtype, head_dim));
    if (workspace_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !workspace))
        return fail(PKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, pl.ws_bytes);

    pkv::AttnParams p{};
    p.out = out;
    p.q = q;
    p.k = k;
    p.v = v;
    p.total_q = total_q;
    p.num_units = units;
    p.max_seqlen_q = max_seqlen_q;
    p.q_heads = q_heads;
    p.kv_heads = kv_heads;
    p.group = group;
    p.causal = causal != 0;
    p.window = w;
    p.kv_start = kv_start;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.row_mode = row_mode ? 1 : 0;
    if (paged) {
        p.mode = pkv::kPagedVarlen;
        p.cu_seqlens_q = cu_seqlens_q;
        p.seqused_k = seqused_k;
        p.block_table = block_table;
        p.max_blocks = max_blocks_per_seq;
        p.num_blocks = num_blocks;
        const int64_t cap64 = (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE;
        p.kv_cap = (int32_t)(cap64 < max_seqlen_k ? cap64 : max_seqlen_k);
    } else {
        p.mode = pkv::kColumn;
        p.seq_info = seq_info;
        p.rows = rows;
        p.cols = cols;
    }
    return run_attention(p, dtype, head_dim, pl, workspace, (hipStream_t)stream);
}

}  // extern "C"
