// Device helpers for gfx950: raw 16-byte loads, bf16 packing, dot2, DPP
// cross-lane reductions on wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

struct alignas(16) u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Nontemporal 16-byte load: for bytes a kernel reads exactly once.
typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(p));
    return u32x4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ void st16(void* p, const u32x4& v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even) and packed, a in the low
// half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f32x2v_t x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v_t));
}

// Packed bf16 pair (1.0, 1.0): dot2 with it sums the pair in fp32.
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

// Round an fp32 value to the nearest bf16 value, kept in fp32.
__device__ __forceinline__ float round_bf16(float f) {
    return __builtin_bit_cast(float, f32_to_bf16_bits(f) << 16);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 inputs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Gather the low (or high) bf16 of two words into one word: lo from a, hi from b.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- DPP lane permutations (all lanes read a valid source) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- 15-i within 16
constexpr int kRowRor4 = 0x124;       // lane i <- (i+4)%16 within a row
constexpr int kRowRor8 = 0x128;       // lane i <- (i+8)%16 within a row

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// A copy of v the compiler cannot see through: the lane-swap builtins below
// are folded wrongly when both of their operands are the same value (the
// second result is taken to equal the first).
__device__ __forceinline__ uint32_t opaque_copy(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}
// op(x, x of lane ^ 32) and op(x, x of lane ^ 16) (op: max or sum) through
// gfx950's v_permlane32_swap / v_permlane16_swap, VALU instructions with no
// LDS round trip.  With x in both operands the two results hold, in every
// lane, x of the lower and of the upper lane of its pair.
template <bool MAX>
__device__ __forceinline__ float swap_op32(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(b, opaque_copy(b), false, false);
    const float lo = __builtin_bit_cast(float, (uint32_t)r[0]), hi = __builtin_bit_cast(float, (uint32_t)r[1]);
    return MAX ? fmaxf(lo, hi) : lo + hi;
}
template <bool MAX>
__device__ __forceinline__ float swap_op16(float x) {
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(b, opaque_copy(b), false, false);
    const float lo = __builtin_bit_cast(float, (uint32_t)r[0]), hi = __builtin_bit_cast(float, (uint32_t)r[1]);
    return MAX ? fmaxf(lo, hi) : lo + hi;
}

// x from lane (lane ^ ST), ST = 1 .. 32.
template <int ST>
__device__ __forceinline__ float xor_lanes(float x) {
    if constexpr (ST == 32) {
        return xor32(x);
    } else {
        // ds_swizzle bitmask mode (within 32-lane halves): and 0x1F, or 0, xor ST
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                                     0x1F | (ST << 10)));
    }
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32, 64);
// every lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<kQuadXor1>(x);
    if constexpr (N >= 4) x += dpp<kQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kRowMirror>(x);
    if constexpr (N >= 32) x = swap_op16<false>(x);
    if constexpr (N >= 64) x = swap_op32<false>(x);
    return x;
}

// Over lanes that share (lane % STRIDE): combine the 64/STRIDE lanes
// l, l+STRIDE, ... (STRIDE = 4, 8, 16, 32, 64); every lane receives the result.
template <int STRIDE, bool MAX>
__device__ __forceinline__ float across_groups(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (STRIDE <= 8) x = op(x, dpp<kRowRor8>(x));
    if constexpr (STRIDE <= 4) x = op(x, dpp<kRowRor4>(x));
    if constexpr (STRIDE <= 16) x = swap_op16<MAX>(x);
    if constexpr (STRIDE <= 32) x = swap_op32<MAX>(x);
    return x;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Two adjacent floats (8-byte aligned) as one device-coherent (agent scope)
// 64-bit store.  On gfx950 this is a plain store with the sc1 scope bit: it
// reaches the coherence point past the per-XCD L2 without the whole-cache
// writeback that a device-scope fence costs.  Used to hand split-K partials
// between work groups.
__device__ __forceinline__ void st_agent2(float* p, float a, float b) {
    const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, a) |
                       ((uint64_t)__builtin_bit_cast(uint32_t, b) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Work-group barrier that orders LDS only: this wave's LDS accesses have
// completed when it passes, while its global loads stay in flight (a full
// __syncthreads() would also wait for those).
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until every vector memory access this wave issued has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- split-K deal over work items, run by one whole wave ----
// Lane l owns items [l*per, min(n_items, (l+1)*per)); item_n(i) is the item's
// work in chunks (>= 0) or -1 when it is not this kernel's.  An item with n
// chunks takes max(1, ceil(n / c)) consecutive slots; deal_size returns the
// smallest c for which all items fit into `slots` (binary search; slots must
// be at least the number of items with work).
__device__ __forceinline__ int32_t deal_slots_of(int32_t n, int32_t c) {
    return n < 0 ? 0 : (n <= c ? 1 : (n + c - 1) / c);
}

// The dealing wave's lane owns items [ib, ie).  Their counts are read once
// (each read is a chain of global loads) and kept in registers for the first
// kDealRegs items; any further items of a lane are read again per pass.
constexpr int kDealRegs = 8;
struct DealItems {
    int32_t ib, ie;
    int32_t n[kDealRegs];
};
template <typename F>
__device__ __forceinline__ DealItems deal_items(const F& item_n, int32_t ib, int32_t ie) {
    DealItems d;
    d.ib = ib;
    d.ie = ie;
#pragma unroll
    for (int k = 0; k < kDealRegs; ++k) d.n[k] = (ib + k < ie) ? item_n(ib + k) : 0;
    return d;
}
// body(item, count) for each of the lane's items, in order.
template <typename F, typename B>
__device__ __forceinline__ void deal_for_each(const DealItems& d, const F& item_n, const B& body) {
#pragma unroll
    for (int k = 0; k < kDealRegs; ++k)
        if (d.ib + k < d.ie) body(d.ib + k, d.n[k]);
    for (int32_t i = d.ib + kDealRegs; i < d.ie; ++i) body(i, item_n(i));
}
// Sum (MAX: maximum) of x over the wave's 64 lanes, wave-uniform: four DPP
// steps within rows of 16 lanes, one swizzle across the two rows of each
// half, and the halves read out of lanes 0 and 32.  No step goes through a
// cross-lane LDS permute (ds_bpermute), whose round trip a chain of six per
// reduction had paid.
template <bool MAX>
__device__ __forceinline__ int32_t wave_reduce_i32(int32_t x) {
    auto op = [](int32_t a, int32_t b) { return MAX ? max(a, b) : a + b; };
    x = op(x, __builtin_amdgcn_update_dpp(0, x, kQuadXor1, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_update_dpp(0, x, kQuadXor2, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_update_dpp(0, x, kRowHalfMirror, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_update_dpp(0, x, kRowMirror, 0xF, 0xF, false));
    x = op(x, __builtin_amdgcn_ds_swizzle(x, 0x401F));
    return op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 32));
}

template <typename F>
__device__ int32_t deal_size(const DealItems& d, const F& item_n, int64_t slots) {
    int32_t nmax = 0;
    deal_for_each(d, item_n, [&](int32_t, int32_t n) { nmax = max(nmax, n); });
    nmax = wave_reduce_i32<true>(nmax);
    int32_t lo = 1, hi = nmax > 1 ? nmax : 1;      // c = nmax gives one slot per item
    // Only whether the count fits `slots` matters (at most the grid's 65535
    // rows): each lane's count saturates at cap, so the wave's sum stays far
    // inside 32 bits whatever the items' sizes.
    const int32_t cap = slots < (1 << 24) ? (int32_t)slots + 1 : (1 << 24);
    while (lo < hi) {                              // wave-uniform loop
        const int32_t c = lo + (hi - lo) / 2;
        int32_t k = 0;
        deal_for_each(d, item_n, [&](int32_t, int32_t n) { k = min(k + deal_slots_of(n, c), cap); });
        k = wave_reduce_i32<false>(k);
        if (k <= slots) hi = c; else lo = c + 1;
    }
    return lo;
}

}  // namespace pkv
