// Batched-sequence column store bookkeeping (host) and the column copy (device).
//
// ExecuTorch PR #24073, the batched-sequence CUDA KV cache: every admitted
// sequence owns one column of a [rows, max_seqs + 1, H, D] store (the last
// column is scratch for padded static-width writes); ring layers hold
// min(capacity, window + max_write - 1) rows, flat layers grow by whole rows;
// the BatchControl surface is declare_step / prepare_step / commit_step,
// seq_clone (a device copy of the source prefix), seq_rm, rewind (bounded by
// the ring floor), pos and max_seqs; prepare_step stages the per-token write
// slots and the seq_info segment table; the token runs of one step are
// validated as one contiguous run per owner.  PR #24076: a ring layer cannot
// wrap before it holds all its rows, so until then it can grow like a flat
// one, capped at its own rows.
//
// The host object never touches device memory: prepare_step fills caller
// host buffers (the caller uploads them), and the device copy of a clone is
// pkv_column_copy, enqueued by the caller.
#include <stdlib.h>

#include <new>
#include <vector>

#include "internal.h"
#include "device_util.h"

struct pkv_batch {
    int32_t max_seqs;
    int32_t capacity;
    int32_t window;
    int32_t max_write;
    int32_t rows;                 // ring rows, or capacity for a flat store
    bool ring;
    std::vector<int32_t> pos;     // per column: next position; -1 when free
    std::vector<int32_t> step_seq, step_n;
    int32_t step_width = 0;
    bool declared = false;
};

namespace {

pkv_status bad(const char* what) {
    pkv::set_error("%s", what);
    return PKV_EINVAL;
}

bool live(const pkv_batch* b, int32_t seq) {
    return b && seq >= 0 && seq < b->max_seqs && b->pos[seq] >= 0;
}

// Lowest position a sequence at `pos` can rewind to: the keys a step
// starting there can see must still be in the ring.
int32_t ring_floor(const pkv_batch* b, int32_t pos) {
    if (!b->ring) return 0;
    const int64_t f = (int64_t)pos - b->rows + b->window - 1;
    return f > 0 ? (int32_t)f : 0;
}

__global__ __launch_bounds__(256) void column_copy_kernel(uint8_t* __restrict__ k, uint8_t* __restrict__ v,
                                                          int64_t row_stride, int64_t col_bytes,
                                                          int32_t src_col, int32_t dst_col,
                                                          int32_t chunks_per_row, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int64_t r = idx / chunks_per_row;
    const int64_t c = idx - r * chunks_per_row;
    const int64_t src = r * row_stride + (int64_t)src_col * col_bytes + c * 16;
    const int64_t dst = r * row_stride + (int64_t)dst_col * col_bytes + c * 16;
    pkv::st16(k + dst, pkv::ld16(k + src));
    pkv::st16(v + dst, pkv::ld16(v + src));
}

}  // namespace

extern "C" {

pkv_batch* pkv_batch_create(int32_t max_seqs, int32_t capacity, int32_t window, int32_t max_write) {
    if (max_seqs <= 0 || capacity <= 0 || max_write <= 0 || window < 0) {
        pkv::set_error("max_seqs, capacity and max_write must be > 0, window >= 0");
        return nullptr;
    }
    pkv_batch* b = new (std::nothrow) pkv_batch;
    if (!b) {
        pkv::set_error("out of host memory");
        return nullptr;
    }
    b->max_seqs = max_seqs;
    b->capacity = capacity;
    b->window = window;
    b->max_write = max_write;
    const int64_t ring_rows = (int64_t)window + max_write - 1;
    b->ring = window > 0 && ring_rows <= capacity;
    b->rows = b->ring ? (int32_t)ring_rows : capacity;
    b->pos.assign(max_seqs, -1);
    return b;
}

void pkv_batch_destroy(pkv_batch* b) { delete b; }

int32_t pkv_batch_max_seqs(const pkv_batch* b) { return b ? b->max_seqs : 0; }
int32_t pkv_batch_cols(const pkv_batch* b) { return b ? b->max_seqs + 1 : 0; }
int32_t pkv_batch_rows(const pkv_batch* b) { return b ? b->rows : 0; }

int32_t pkv_batch_rows_needed(const pkv_batch* b, int32_t step_width, int32_t row_step) {
    if (!b || step_width < 0 || row_step <= 0) return 0;
    int64_t need = step_width;                 // the scratch column's padded writes
    for (int32_t s = 0; s < b->max_seqs; ++s)
        if (b->pos[s] >= 0) need = need > (int64_t)b->pos[s] + step_width ? need : (int64_t)b->pos[s] + step_width;
    need = (need + row_step - 1) / row_step * row_step;
    return (int32_t)(need < b->rows ? need : b->rows);
}

pkv_status pkv_batch_seq_new(pkv_batch* b, int32_t* seq) {
    if (!b || !seq) return bad("null argument");
    if (b->declared) return bad("a step is declared: commit it first");
    for (int32_t s = 0; s < b->max_seqs; ++s)
        if (b->pos[s] < 0) {
            b->pos[s] = 0;
            *seq = s;
            pkv::clear_error();
            return PKV_OK;
        }
    return bad("every column holds a sequence");
}

pkv_status pkv_batch_seq_rm(pkv_batch* b, int32_t seq) {
    if (!live(b, seq)) return bad("no such sequence");
    if (b->declared) return bad("a step is declared: commit it first");
    b->pos[seq] = -1;
    pkv::clear_error();
    return PKV_OK;
}

pkv_status pkv_batch_seq_clone(pkv_batch* b, int32_t src, int32_t* dst, int32_t* copy_rows) {
    if (!live(b, src) || !dst || !copy_rows) return bad("no such sequence or null argument");
    int32_t d = -1;
    pkv_status s = pkv_batch_seq_new(b, &d);
    if (s != PKV_OK) return s;
    b->pos[d] = b->pos[src];
    *dst = d;
    *copy_rows = b->pos[src] < b->rows ? b->pos[src] : b->rows;
    return PKV_OK;
}

pkv_status pkv_batch_rewind(pkv_batch* b, int32_t seq, int32_t pos) {
    if (!live(b, seq)) return bad("no such sequence");
    if (b->declared) return bad("a step is declared: commit it first");
    if (pos > b->pos[seq]) return bad("rewind past the current position");
    if (pos < ring_floor(b, b->pos[seq])) return bad("rewind below the ring floor");
    b->pos[seq] = pos;
    pkv::clear_error();
    return PKV_OK;
}

pkv_status pkv_batch_pos(const pkv_batch* b, int32_t seq, int32_t* pos) {
    if (!live(b, seq) || !pos) return bad("no such sequence or null argument");
    *pos = b->pos[seq];
    return PKV_OK;
}

int32_t pkv_batch_floor(const pkv_batch* b, int32_t seq) {
    return live(b, seq) ? ring_floor(b, b->pos[seq]) : -1;
}

pkv_status pkv_batch_declare_step(pkv_batch* b, const int32_t* seqs, const int32_t* n_tokens,
                                  int32_t count, int32_t width) {
    if (!b || (count > 0 && (!seqs || !n_tokens))) return bad("null argument");
    if (count < 0 || count > b->max_seqs) return bad("count out of range");
    std::vector<char> seen(b->max_seqs, 0);
    int64_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        const int32_t s = seqs[i], n = n_tokens[i];
        if (!live(b, s)) return bad("step names a sequence that does not exist");
        if (seen[s]) return bad("a sequence owns more than one run of the step");
        seen[s] = 1;
        if (n < 1 || n > b->max_write) return bad("tokens per sequence must be in 1 .. max_write");
        if (!b->ring && (int64_t)b->pos[s] + n > b->capacity) return bad("a flat column is full");
        total += n;
    }
    if (width < total || width > 1 << 24) return bad("step width below the tokens declared");
    b->step_seq.assign(seqs, seqs + count);
    b->step_n.assign(n_tokens, n_tokens + count);
    b->step_width = width;
    b->declared = true;
    pkv::clear_error();
    return PKV_OK;
}

pkv_status pkv_batch_prepare_step(pkv_batch* b, int32_t* seq_info, int32_t max_segments, int64_t* slots,
                                  int32_t* num_segments) {
    if (!b || !seq_info || !slots || !num_segments) return bad("null argument");
    if (!b->declared) return bad("no step declared");
    const int32_t count = (int32_t)b->step_seq.size();
    if (max_segments < count) return bad("seq_info has fewer rows than the step's sequences");
    const int64_t cols = (int64_t)b->max_seqs + 1;
    int32_t q = 0;
    for (int32_t i = 0; i < count; ++i) {
        const int32_t s = b->step_seq[i], n = b->step_n[i], p0 = b->pos[s];
        seq_info[4 * i + 0] = q;
        seq_info[4 * i + 1] = n;
        seq_info[4 * i + 2] = s;
        seq_info[4 * i + 3] = p0 + n;
        for (int32_t t = 0; t < n; ++t) slots[q + t] = (int64_t)((p0 + t) % b->rows) * cols + s;
        q += n;
    }
    for (int32_t i = count; i < max_segments; ++i)      // segments with no rows
        seq_info[4 * i + 0] = seq_info[4 * i + 1] = seq_info[4 * i + 2] = seq_info[4 * i + 3] = 0;
    for (int32_t t = q; t < b->step_width; ++t)          // padding: the scratch column
        slots[t] = (int64_t)((t - q) % b->rows) * cols + b->max_seqs;
    *num_segments = count;
    pkv::clear_error();
    return PKV_OK;
}

pkv_status pkv_batch_commit_step(pkv_batch* b) {
    if (!b || !b->declared) return bad("no step declared");
    for (size_t i = 0; i < b->step_seq.size(); ++i) b->pos[b->step_seq[i]] += b->step_n[i];
    b->step_seq.clear();
    b->step_n.clear();
    b->declared = false;
    pkv::clear_error();
    return PKV_OK;
}

pkv_status pkv_column_copy(void* k, void* v, int32_t rows, int32_t cols, int32_t kv_heads, int32_t head_dim,
                           int32_t src_col, int32_t dst_col, int32_t n_rows, pkv_dtype dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16) return bad("unknown dtype");
    if (rows <= 0 || cols <= 0 || kv_heads <= 0 || head_dim <= 0 || head_dim % 8 != 0)
        return bad("rows, cols, kv_heads must be > 0 and head_dim a positive multiple of 8");
    if (src_col < 0 || src_col >= cols || dst_col < 0 || dst_col >= cols) return bad("column out of range");
    if (n_rows < 0 || n_rows > rows) return bad("n_rows out of range");
    if (n_rows == 0 || src_col == dst_col) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k || !v) return bad("null pointer argument");
    if (((uintptr_t)k & 15) || ((uintptr_t)v & 15)) return bad("store pointers must be 16-byte aligned");
    const int64_t col_bytes = (int64_t)kv_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4);
    const int32_t cpr = (int32_t)(col_bytes / 16);
    const int64_t total = (int64_t)n_rows * cpr;
    const int64_t grid = (total + 255) / 256;
    column_copy_kernel<<<dim3((uint32_t)grid), dim3(256), 0, (hipStream_t)stream>>>(
        (uint8_t*)k, (uint8_t*)v, col_bytes * cols, col_bytes, src_col, dst_col, cpr, total);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("column_copy: %s", hipGetErrorString(e));
        return PKV_EHIP;
    }
    pkv::clear_error();
    return PKV_OK;
}

}  // extern "C"
