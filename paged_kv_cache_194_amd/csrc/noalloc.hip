// pkv_paged_decode_attn_noalloc: single-query paged decode for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The split-K scratch that pkv_paged_decode_attn takes as a caller workspace
// is here a static device array of PKV_NOALLOC_SCRATCH_BYTES: each GPU the
// library runs on holds its own copy until the process ends.  In host code the
// array's name stands for a host-side shadow, not a device address, so it is
// never passed to a kernel or a copy: its address on each device is looked up
// once, with that device current, and kept.
#include <mutex>

#include "internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on device d

// Device address of `scratch` on the current device (looked up on the first
// call there).
pkv_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        pkv::set_error("hipGetDevice: %s", hipGetErrorString(e));
        return PKV_EHIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        pkv::set_error("device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
        return PKV_EUNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            pkv::set_error("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            return PKV_EHIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PKV_OK;
}

// Zero n16 16-byte words: a kernel rather than hipMemsetAsync, so that a call
// captured into a graph clears the counters on every replay.
__global__ __launch_bounds__(256) void clear16_kernel(uint4* p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_attn_noalloc(
    void* out, const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
    int32_t block_size, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* seqused_k, int32_t num_seqs, int32_t max_seqlen_k, const void* k_new,
    const void* v_new, int32_t q_heads, int32_t kv_heads, int32_t head_dim, float softmax_scale,
    int32_t causal, int32_t window, const int32_t* kv_start, int32_t num_splits, pkv_dtype dtype,
    void* stream) {
    size_t need = 0, tickets = 0;
    pkv_status s = pkv::decode_check(out, q, k_cache, v_cache, num_blocks, block_size, block_table,
                                     max_blocks_per_seq, seqused_k, num_seqs, max_seqlen_k, k_new, v_new,
                                     q_heads, kv_heads, head_dim, softmax_scale, num_splits, dtype, &need,
                                     &tickets);
    if (s != PKV_OK) return s;
    if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) {
        pkv::set_error("this call needs %zu bytes of split-K scratch; the static scratch holds %zu "
                       "(pass fewer num_splits, or use pkv_paged_decode_attn with a workspace)",
                       need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
        return PKV_EWORKSPACE;
    }
    void* ws = nullptr;
    if (num_seqs > 0 && need > 0) {
        s = scratch_address(&ws);
        if (s != PKV_OK) return s;
        // The array keeps whatever the last call on this device left, and a
        // call of another shape may have put partials where this call's
        // arrival counters sit: clear them first.
        if (tickets > 0) {
            const int64_t n16 = (int64_t)(tickets / 16);
            const int blocks = (int)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
            clear16_kernel<<<dim3(blocks), dim3(256), 0, (hipStream_t)stream>>>((uint4*)ws, n16);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) {
                pkv::set_error("clearing the scratch counters: %s", hipGetErrorString(e));
                return PKV_EHIP;
            }
        }
    }
    return pkv_paged_decode_attn(out, q, k_cache, v_cache, num_blocks, block_size, block_table,
                                 max_blocks_per_seq, seqused_k, num_seqs, max_seqlen_k, k_new, v_new,
                                 q_heads, kv_heads, head_dim, softmax_scale, causal, window, kv_start,
                                 num_splits, ws, (size_t)PKV_NOALLOC_SCRATCH_BYTES, dtype, stream);
}
