// Internal interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// How a unit (a sequence or a segment) finds its query rows and keys.
enum AddrMode : int32_t {
    kPagedDecode = 0,   // one query row per sequence, row b; block table
    kPagedVarlen = 1,   // rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; block table
    kColumn = 2,        // seq_info (q_start, q_len, col, kv_end); ring column store
};

// Everything an attention kernel reads, passed by value.
struct AttnParams {
    void* out;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* cu_seqlens_q;
    const int32_t* seqused_k;
    const int32_t* block_table;
    const int32_t* seq_info;
    const int32_t* kv_start;   // left-padding bound per unit, or null (none)
    const void* k_new;     // fused append (paged decode): [units, Hkv, D] or null
    const void* v_new;
    float* ws_o;           // split-K partial outputs [vec_wgs][Hkv][GT][D]
    float* ws_ml;          // split-K partial (max, sum) [vec_wgs][Hkv][GT][2]
    int32_t* ws_ticket;    // per (unit, kv head) arrival counters, zero between calls
    float* mws_o;          // matrix-core path partials [units*Hkv*tiles*splits][BM][D]
    float* mws_ml;         // and their (max, sum) [..][BM][2]
    int32_t* mws_ticket;   // per (unit, kv head, tile) arrival counters
    int32_t mfma_tiles;    // row tiles per (unit, kv head) on the matrix-core path
    int32_t mfma_splits;
    int32_t mode;
    int32_t total_q;
    int32_t num_units;
    int32_t max_blocks;    // block-table row width (paged)
    int32_t num_blocks;    // pool blocks (paged)
    int32_t rows;          // ring rows (column)
    int32_t cols;          // store columns (column)
    int32_t max_seqlen_q;
    int32_t kv_cap;        // clamp for seqused_k (paged)
    int32_t q_heads;
    int32_t kv_heads;
    int32_t group;         // q_heads / kv_heads
    int32_t causal;
    int32_t window;
    int32_t num_splits;    // vector path: split-K partitions per unit (on average)
    int32_t vec_wgs;       // vector path: work-group slots per kv head
    int32_t vec_units;     // vector path: work items (units, or unit rows in row mode)
    int32_t row_mode;      // vector path takes each row of a unit as its own item
    int32_t mfma_single;   // matrix-core path takes single-row units too (no vector launch)
    int32_t zero_rows;     // the attention launch also zeroes the rows no unit covers
    float scale_log2;      // softmax_scale * log2(e)
};

// Where one unit's rows and keys are, resolved on the device.
struct UnitInfo {
    int32_t q_start;
    int32_t q_len;
    int32_t kv_end;        // E after clamping
    int32_t col;           // column mode only
    int32_t pad;           // left-padding bound (kv_start); <= 0: none
    bool keys_ok;          // column inside the store (column mode); true otherwise
};

__device__ __forceinline__ UnitInfo load_unit(const AttnParams& p, int32_t u) {
    UnitInfo ui;
    ui.col = 0;
    ui.keys_ok = true;
    ui.pad = p.kv_start ? p.kv_start[u] : 0;
    if (p.mode == kColumn) {
        const int32_t* s = p.seq_info + 4 * (int64_t)u;
        ui.q_start = s[0];
        ui.q_len = s[1];
        ui.col = s[2];
        ui.kv_end = s[3] < 0 ? 0 : s[3];
        ui.keys_ok = (ui.col >= 0) && (ui.col < p.cols);
    } else {
        if (p.mode == kPagedDecode) {
            ui.q_start = u;
            ui.q_len = 1;
        } else {
            ui.q_start = p.cu_seqlens_q[u];
            ui.q_len = p.cu_seqlens_q[u + 1] - ui.q_start;
        }
        int32_t e = p.seqused_k[u];
        ui.kv_end = e < 0 ? 0 : (e > p.kv_cap ? p.kv_cap : e);
    }
    return ui;
}

// Key range [lo, hi) of the first query row of a unit of L rows over E keys,
// the row the vector path computes: the unit's only row, or row 0 when the
// call's static bound max_seqlen_q is 1 (later rows are then uncovered).  The
// row sits at position pos = E - L (tiny-llm kv_cache.py, causal_kwargs:
// bottom-right alignment).  Causal: keys up to pos; window W: the W keys
// ending at pos; left-padding bound pad > 0: no key before it, and a row
// before it (a pad query) keeps only its own key (padded_causal_mask).
struct KeyRange {
    int32_t lo, hi;
};
__device__ __forceinline__ KeyRange first_row_keys(const AttnParams& p, int32_t E, int32_t L, int32_t pad) {
    const int32_t pos = E - L;
    KeyRange r;
    if (pad > 0 && pos < pad) {
        r.lo = pos > 0 ? pos : 0;
        r.hi = pos + 1 < E ? pos + 1 : E;
    } else {
        r.hi = p.causal ? (pos + 1 < E ? pos + 1 : E) : E;
        r.lo = (p.window > 0 && pos - p.window + 1 > 0) ? pos - p.window + 1 : 0;
        if (pad > r.lo) r.lo = pad;
    }
    if (r.hi < r.lo) r.hi = r.lo;
    return r;
}

// The host checks of pkv_paged_decode_attn, without enqueuing anything; on
// PKV_OK also the workspace bytes the call needs and how many of them, at the
// start, hold split-K arrival counters.
pkv_status decode_check(void* out, const void* q, const void* k_cache, const void* v_cache,
                        int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* seqused_k, int32_t num_seqs,
                        int32_t max_seqlen_k, const void* k_new, const void* v_new,
                        int32_t q_heads, int32_t kv_heads, int32_t head_dim, float softmax_scale,
                        int32_t num_splits, pkv_dtype dtype, size_t* ws_bytes, size_t* ticket_bytes);

// Zero the output rows [r0, r0 + n) (n <= 32) that no unit covers, run by a
// whole work group of `nthreads` threads: wave 0 reads the units' row ranges
// 64 per vector load and marks each covered row with one ballot, then every
// thread clears uncovered rows 16 bytes at a time.  *todo is an LDS word.
// Rows of a unit past max_seqlen_q count as uncovered.
__device__ __forceinline__ void zero_uncovered_rows(const AttnParams& p, int32_t r0, int32_t n,
                                                    int32_t row_bytes, uint32_t* todo, int nthreads) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t cov = 0;                           // bit i: row r0 + i is covered
        for (int32_t ub = 0; ub < p.num_units; ub += 64) {
            const int32_t u = ub + lane;
            int32_t q0 = 0, L = 0;
            if (u < p.num_units) {
                if (p.mode == kColumn) {
                    q0 = p.seq_info[4 * (int64_t)u];
                    L = p.seq_info[4 * (int64_t)u + 1];
                } else if (p.mode == kPagedVarlen) {
                    q0 = p.cu_seqlens_q[u];
                    L = p.cu_seqlens_q[u + 1] - q0;
                } else {
                    q0 = u;
                    L = 1;
                }
                if (L > p.max_seqlen_q) L = p.max_seqlen_q;
            }
            for (int i = 0; i < n; ++i) {
                const int32_t r = r0 + i;
                if (__ballot(r >= q0 && r - q0 < L) != 0) cov |= 1u << i;
            }
        }
        if (lane == 0) {
            const uint32_t inside = n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
            *todo = ~cov & inside;
        }
    }
    __syncthreads();
    const uint32_t t = *todo;
    if (t == 0) return;
    const int32_t chunks = row_bytes / 16;
    for (int32_t i = threadIdx.x; i < n * chunks; i += nthreads) {
        const int32_t rr = i / chunks, c = i - rr * chunks;
        if ((t >> rr) & 1u)
            *reinterpret_cast<uint4*>((uint8_t*)p.out + (int64_t)(r0 + rr) * row_bytes + (int64_t)c * 16) =
                make_uint4(0u, 0u, 0u, 0u);
    }
}

// Uncovered-row zeroing inside an attention launch: the work groups of kv
// head 0 (blockIdx.x == 0) each take an equal share of the rows, 32 at a
// time, before their attention work (a separate column of work groups could
// push a grid of one work group per CU into a second dispatch round).
__device__ __forceinline__ void zero_rows_share(const AttnParams& p, int32_t row_bytes, uint32_t* todo,
                                                int nthreads) {
    const int64_t zi = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    const int64_t nz = (int64_t)gridDim.y * gridDim.z;
    const int64_t per = ((int64_t)p.total_q + nz - 1) / nz;
    const int64_t end = (zi + 1) * per < p.total_q ? (zi + 1) * per : p.total_q;
    for (int64_t r0 = zi * per; r0 < end; r0 += 32)
        zero_uncovered_rows(p, (int32_t)r0, (int32_t)(end - r0 < 32 ? end - r0 : 32), row_bytes, todo, nthreads);
}

// Text for pkv_last_error() on the calling thread.
void set_error(const char* fmt, ...);
void clear_error();

// ---- launchers (each returns hipGetLastError() of its launch) ----

hipError_t launch_kv_append(void* k_cache, void* v_cache, int64_t num_slots,
                            const void* k_new, const void* v_new, int32_t num_tokens,
                            const int64_t* slot_mapping, int64_t row_bytes, hipStream_t stream);

// Single-query decode append with the slot found on the device: row b of
// k_new/v_new to position clamp(seqused_k[b], 0, kv_cap) - 1 through the block
// table; nothing for an empty sequence or an entry outside the pool.
hipError_t launch_decode_append(void* k_cache, void* v_cache, int32_t num_blocks, const void* k_new,
                                const void* v_new, int32_t num_seqs, int64_t row_bytes,
                                const int32_t* seqused_k, int32_t kv_cap, const int32_t* block_table,
                                int32_t max_blocks, hipStream_t stream);

// Prefix copies between a dense [batch, heads, src_len, D] cache and paged
// slots; to_dense = export (then src_len == n and seqused_k is unused).
hipError_t launch_prefix_copy(bool to_dense, void* dst_k, void* dst_v, const void* src_k,
                              const void* src_v, const int32_t* block_table, int32_t max_blocks,
                              int32_t num_blocks, int32_t batch, int32_t n, int32_t src_len,
                              int32_t heads, int64_t row_bytes, int32_t* seqused_k,
                              hipStream_t stream);

// Vector-ALU path for units with one query row (q_len == 1) and group <= 8
// (the library routes bf16 groups of 8 to the matrix cores; the kernel takes
// them too).  Returns hipErrorInvalidValue when no kernel is compiled for (dtype, D, group).
hipError_t launch_attn_vec(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                           hipStream_t stream);
bool attn_vec_supported(pkv_dtype dtype, int32_t head_dim, int32_t group);

// Matrix-core path for units with several query rows, and single-row units
// with a group of 8 or more: bf16.
hipError_t launch_attn_mfma(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                            hipStream_t stream);
bool attn_mfma_supported(pkv_dtype dtype, int32_t head_dim);
// Shape figures of the matrix-core launch for a call whose units have up to
// `rows` = max_seqlen_q * group rows: rows per work group, keys per chunk,
// work groups per CU.
int32_t mfma_rows_per_group(int32_t head_dim, int64_t rows);
int32_t mfma_chunk_keys(int32_t head_dim, int64_t rows);
int32_t mfma_groups_per_cu(int32_t head_dim, int64_t rows);

// Zero every output row of [0, total_q) that no unit covers.
hipError_t launch_zero_uncovered(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                                 hipStream_t stream);

// Rows of query a vector-path work group holds (group size rounded up).
int32_t vec_group_rows(int32_t group);

// Arrival counters of split-K sit one per 256 bytes, so that the work groups
// of different heads do not queue on one memory line.
constexpr int32_t kTicketStride = 64;

// Bytes of the arrival counters at the start of a split-K workspace.
size_t ticket_bytes(int32_t units, int32_t kv_heads);

// Work-group slots per kv head of the vector path for `units` units at
// `splits` partitions per unit.
int32_t vec_slots(int32_t units, int32_t splits);

}  // namespace pkv
