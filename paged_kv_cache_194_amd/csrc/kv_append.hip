// K/V append: raw 16-byte copies of new token rows into cache slots.
//
// vLLM-Omni paged_decode, PagedDecodeCache.attend: this step's K and V go into
// the flat slot view (num_blocks * 16, kv_heads, head_dim) at a slot held in a
// device tensor, so a replayed graph writes the slot current at replay time.
// ExecuTorch PR #24073: the column store takes in-graph writes at slot
// (position % rows) * columns + column; the caller hands either slot in.
#include "internal.h"
#include "device_util.h"

namespace pkv {

// One thread moves one 16-byte chunk of one token's K row and V row.
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int64_t num_slots,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new, int64_t total_chunks,
    int32_t chunks_per_row, const int64_t* __restrict__ slot_mapping) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total_chunks) return;
    const int64_t t = idx / chunks_per_row;
    const int32_t c = (int32_t)(idx - t * chunks_per_row);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    const int64_t src = t * row_bytes + (int64_t)c * 16;
    const int64_t dst = slot * row_bytes + (int64_t)c * 16;
    st16(k_cache + dst, ld16(k_new + src));
    st16(v_cache + dst, ld16(v_new + src));
}

// Append for single-query decode, slot found on the device: sequence b's new
// row goes to position seqused_k[b] - 1 (clamped like the attention's length)
// through its block-table row, as PagedDecodeCache.attend writes this step's
// K/V before attending.  A sequence with no live key, or whose entry lies
// outside the pool, writes nothing.  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void decode_append_kernel(
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, int32_t num_blocks,
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new, int32_t num_seqs,
    int32_t chunks_per_row, const int32_t* __restrict__ seqused_k, int32_t kv_cap,
    const int32_t* __restrict__ block_table, int32_t max_blocks) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)num_seqs * chunks_per_row) return;
    const int32_t b = (int32_t)(idx / chunks_per_row);
    const int32_t c = (int32_t)(idx - (int64_t)b * chunks_per_row);
    int32_t e = seqused_k[b];
    e = e < 0 ? 0 : (e > kv_cap ? kv_cap : e);
    if (e == 0) return;
    const int32_t pos = e - 1;
    const int32_t id = block_table[(int64_t)b * max_blocks + (pos >> 4)];
    if (id < 0 || id >= num_blocks) return;
    const int64_t row_bytes = (int64_t)chunks_per_row * 16;
    const int64_t dst = ((int64_t)id * 16 + (pos & 15)) * row_bytes + (int64_t)c * 16;
    const int64_t src = (int64_t)b * row_bytes + (int64_t)c * 16;
    st16(k_cache + dst, ld16(k_new + src));
    st16(v_cache + dst, ld16(v_new + src));
}

hipError_t launch_decode_append(void* k_cache, void* v_cache, int32_t num_blocks, const void* k_new,
                                const void* v_new, int32_t num_seqs, int64_t row_bytes,
                                const int32_t* seqused_k, int32_t kv_cap, const int32_t* block_table,
                                int32_t max_blocks, hipStream_t stream) {
    const int32_t cpr = (int32_t)(row_bytes / 16);
    const int64_t total = (int64_t)num_seqs * cpr;
    decode_append_kernel<<<dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream>>>(
        (uint8_t*)k_cache, (uint8_t*)v_cache, num_blocks, (const uint8_t*)k_new, (const uint8_t*)v_new,
        num_seqs, cpr, seqused_k, kv_cap, block_table, max_blocks);
    return hipGetLastError();
}

hipError_t launch_kv_append(void* k_cache, void* v_cache, int64_t num_slots,
                            const void* k_new, const void* v_new, int32_t num_tokens,
                            const int64_t* slot_mapping, int64_t row_bytes, hipStream_t stream) {
    const int32_t cpr = (int32_t)(row_bytes / 16);
    const int64_t total = (int64_t)num_tokens * cpr;
    const int64_t grid = (total + 255) / 256;
    kv_append_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(
        (uint8_t*)k_cache, (uint8_t*)v_cache, num_slots, (const uint8_t*)k_new,
        (const uint8_t*)v_new, total, cpr, slot_mapping);
    return hipGetLastError();
}

}  // namespace pkv
