// Vector-ALU decode attention: units with one query row, GQA group <= 8.
//
// What it computes (vLLM-Omni paged_decode, PagedDecodeCache.attend calling
// flash_attn_varlen_func with max_seqlen_q = 1; ExecuTorch PR #24073 for
// sdpa_varlen's column store, window, zeroed rows and split-K): for the query
// row of a unit and each q head h of kv head g, softmax(q_h . K^T * scale) V
// over the unit's visible live keys, read through the block table or ring.
//
// Work decomposition: one work group (4 waves) per (split, kv head, unit).  The
// unit's visible keys, taken as whole 16-token blocks, are cut into `splits`
// contiguous block ranges; wave w of a work group takes blocks w, w+4, ... of
// its range, so the reduction order depends only on logical positions (a
// permuted block table gives bit-identical results).
//
// Per block a wave holds the 16 tokens' K for its kv head in registers laid
// out KLPT lanes per token (so q . k needs only a KLPT-lane DPP reduction), and
// their V laid out one 16-byte chunk per lane.  All G query heads of the group
// are scored against the same registers (GQA sharing).  Scores go through an
// online softmax (running max per head, wave-uniform after a cross-lane max);
// the probabilities move from the K layout to the V layout through a small
// per-wave LDS slab.  bf16 inputs use v_dot2_f32_bf16 for both products, with
// the probabilities rounded to bf16 (the sum l uses the same rounded values, so
// a constant V comes back exactly).  Accumulation is fp32.
//
// Keys outside the visible range never reach the sums: their scores become
// -inf by selection and their V chunks are replaced by 0, so NaN or Inf
// garbage in the storage past seqused_k cannot leak.
#include "internal.h"
#include "device_util.h"

namespace pkv {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <typename T, int D, int GT>
struct VecCfg {
    static constexpr bool kBF16 = sizeof(T) == 2;
    static constexpr int EB = sizeof(T);
    static constexpr int VEC = 16 / EB;       // elements per 16-byte chunk
    static constexpr int RC = D / VEC;        // chunks per token row of one head
    static constexpr int qdw(int klpt) { return GT * (RC / klpt) * 4; }
    // Lanes per token in the K layout: the fewest that keep q in <= 64 dwords.
    static constexpr int KLPT = (RC >= 4 && qdw(4) <= 64) ? 4
                              : (RC >= 8 && qdw(8) <= 64) ? 8
                              : (RC >= 16 && qdw(16) <= 64) ? 16
                              : (RC >= 32 && qdw(32) <= 64) ? 32 : RC;
    static constexpr int KCH = RC / KLPT;     // chunks per lane per token
    static constexpr int KTPW = 64 / KLPT;    // tokens per wave-wide load
    static constexpr int KNI = 16 / KTPW;     // loads per 16-token block
    static constexpr int VLPT = RC < 64 ? RC : 64;
    static constexpr int VTPW = 64 / VLPT;
    static constexpr int VNI = 16 / VTPW;
    static_assert(KTPW <= 16 && KNI * KTPW == 16, "K layout must tile a block");
    static_assert(VTPW <= 16 && VNI * VTPW == 16, "V layout must tile a block");
    static_assert(!kBF16 || (VNI % 2 == 0), "bf16 PV pairs tokens");
};

template <typename T, int D, int GT>
__global__ __launch_bounds__(kThreads) void attn_vec_kernel(AttnParams p) {
    using C = VecCfg<T, D, GT>;
    constexpr int EB = C::EB, VEC = C::VEC, KLPT = C::KLPT, KCH = C::KCH, KTPW = C::KTPW,
                  KNI = C::KNI, VLPT = C::VLPT, VTPW = C::VTPW, VNI = C::VNI;

    __shared__ float sP[kWaves][16 * GT];
    __shared__ float sO[kWaves][GT][D];
    __shared__ float sM[kWaves][GT];
    __shared__ float sL[kWaves][GT];

    const int32_t split = blockIdx.x;
    const int32_t g = blockIdx.y;
    const int32_t u = blockIdx.z;
    const UnitInfo ui = load_unit(p, u);
    if (ui.q_len != 1) return;                      // other units are not this path's
    const int32_t row = ui.q_start;
    if (row < 0 || row >= p.total_q) return;

    const int32_t G = p.group;
    const int32_t Hkv = p.kv_heads;
    const int32_t S = p.num_splits;
    const int32_t E = ui.keys_ok ? ui.kv_end : 0;
    // One query at position E-1: keys [lo, E) with the window's lower bound.
    const int32_t lo = (p.window > 0 && E - p.window > 0) ? E - p.window : 0;
    const int32_t hi = E;
    const int32_t b_first = lo >> 4;
    const int32_t b_end = (hi + 15) >> 4;
    const int32_t nblk = b_end > b_first ? b_end - b_first : 0;
    const int32_t bps = (nblk + S - 1) / S;
    const int32_t sb = b_first + split * bps;
    const int32_t se = min(b_end, sb + bps);

    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int kpart = lane % KLPT, ktok = lane / KLPT;
    const int vpart = lane % VLPT, vtok = lane / VLPT;

    const uint8_t* __restrict__ Kb = (const uint8_t*)p.k;
    const uint8_t* __restrict__ Vb = (const uint8_t*)p.v;
    const int64_t tok_stride = (int64_t)Hkv * D * EB;        // bytes between tokens of a block
    const int64_t head_off = (int64_t)g * D * EB;

    // q of the group's heads in the K layout: chunk kpart + KLPT*c of each head.
    u32x4 qr[GT][KCH];
    {
        const uint8_t* qb = (const uint8_t*)p.q + ((int64_t)row * p.q_heads + (int64_t)g * G) * D * EB;
#pragma unroll
        for (int r = 0; r < GT; ++r)
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                if (r < G) qr[r][c] = ld16(qb + (int64_t)r * D * EB + (kpart + KLPT * c) * 16);
                else qr[r][c] = u32x4{0u, 0u, 0u, 0u};
            }
    }

    float m[GT], l[GT], acc[GT][VEC];
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][e] = 0.f;
    }

    for (int32_t blk = sb + wave; blk < se; blk += kWaves) {
        const int32_t t0 = blk * 16;
        // ---- storage of this block ----
        int64_t pbase = 0;
        int32_t row0 = 0;
        if (p.mode == kColumn) {
            row0 = t0 % p.rows;
        } else {
            const int32_t id = p.block_table[(int64_t)u * p.max_blocks + blk];
            if (id < 0 || id >= p.num_blocks) continue;      // no storage: keys contribute nothing
            pbase = (int64_t)id * 16 * tok_stride + head_off;
        }
        auto tok_addr = [&](int tt) -> int64_t {
            if (p.mode == kColumn) {
                int32_t r = row0 + tt;
                if (r >= p.rows) r -= p.rows;
                if (r >= p.rows) r %= p.rows;       // rings shorter than a block
                return ((int64_t)r * p.cols + ui.col) * tok_stride + head_off;
            }
            return pbase + (int64_t)tt * tok_stride;
        };

        u32x4 kr[KNI][KCH];
        u32x4 vr[VNI];
#pragma unroll
        for (int i = 0; i < KNI; ++i) {
            const int64_t a = tok_addr(i * KTPW + ktok);
#pragma unroll
            for (int c = 0; c < KCH; ++c) kr[i][c] = ld16(Kb + a + (kpart + KLPT * c) * 16);
        }
#pragma unroll
        for (int i = 0; i < VNI; ++i) vr[i] = ld16(Vb + tok_addr(i * VTPW + vtok) + vpart * 16);

        const bool full = (t0 >= lo) && (t0 + 16 <= hi);

        // ---- scores for every head of the group (all lanes of a token agree) ----
        float s[KNI][GT];
#pragma unroll
        for (int i = 0; i < KNI; ++i) {
            const int32_t t = t0 + i * KTPW + ktok;
            const bool vis = full || (t >= lo && t < hi);
#pragma unroll
            for (int r = 0; r < GT; ++r) {
                float d = 0.f;
#pragma unroll
                for (int c = 0; c < KCH; ++c) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        if constexpr (C::kBF16) {
                            d = dot2_bf16(word(qr[r][c], w), word(kr[i][c], w), d);
                        } else {
                            d = fmaf(__builtin_bit_cast(float, word(qr[r][c], w)),
                                     __builtin_bit_cast(float, word(kr[i][c], w)), d);
                        }
                    }
                }
                d = group_sum<KLPT>(d) * p.scale_log2;
                s[i][r] = vis ? d : -INFINITY;
            }
        }

        // ---- online softmax: per-head block max, rescale factor, probabilities ----
        float alpha[GT];
        bool rescale = false;
#pragma unroll
        for (int r = 0; r < GT; ++r) {
            float mb = s[0][r];
#pragma unroll
            for (int i = 1; i < KNI; ++i) mb = fmaxf(mb, s[i][r]);
            mb = across_groups<KLPT, true>(mb);
            const float m_new = fmaxf(m[r], mb);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[r] = fast_exp2(m[r] - m_use);
            rescale |= (m_new != m[r]);
            m[r] = m_new;
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < KNI; ++i) {
                float pr = fast_exp2(s[i][r] - m_use);
                if constexpr (C::kBF16) pr = round_bf16(pr);
                s[i][r] = pr;
                ps += pr;
            }
            l[r] = l[r] * alpha[r] + ps;
        }

        // ---- probabilities from the K layout to the V layout through LDS ----
        float* P = sP[wave];
        if (kpart == 0) {
#pragma unroll
            for (int i = 0; i < KNI; ++i)
#pragma unroll
                for (int r = 0; r < GT; ++r) P[(i * KTPW + ktok) * GT + r] = s[i][r];
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        float pv[VNI][GT];
#pragma unroll
        for (int i = 0; i < VNI; ++i)
#pragma unroll
            for (int r = 0; r < GT; ++r) pv[i][r] = P[(i * VTPW + vtok) * GT + r];
        __atomic_signal_fence(__ATOMIC_SEQ_CST);

        if (rescale) {   // wave-uniform: m is identical in every lane
#pragma unroll
            for (int r = 0; r < GT; ++r)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[r][e] *= alpha[r];
        }

        if (!full) {
#pragma unroll
            for (int i = 0; i < VNI; ++i) {
                const int32_t t = t0 + i * VTPW + vtok;
                if (!(t >= lo && t < hi)) vr[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }

        // ---- PV ----
        if constexpr (C::kBF16) {
#pragma unroll
            for (int i = 0; i < VNI; i += 2) {
                uint32_t vp[VEC];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    vp[2 * w] = pair_lo(word(vr[i], w), word(vr[i + 1], w));
                    vp[2 * w + 1] = pair_hi(word(vr[i], w), word(vr[i + 1], w));
                }
#pragma unroll
                for (int r = 0; r < GT; ++r) {
                    const uint32_t pp = pair_hi(__builtin_bit_cast(uint32_t, pv[i][r]),
                                                __builtin_bit_cast(uint32_t, pv[i + 1][r]));
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[r][e] = dot2_bf16(pp, vp[e], acc[r][e]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < VNI; ++i)
#pragma unroll
                for (int r = 0; r < GT; ++r)
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        acc[r][e] = fmaf(pv[i][r], __builtin_bit_cast(float, word(vr[i], e)), acc[r][e]);
        }
    }

    // ---- merge lanes, then waves ----
#pragma unroll
    for (int r = 0; r < GT; ++r) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][e] = across_groups<VLPT, false>(acc[r][e]);
        l[r] = across_groups<KLPT, false>(l[r]);
    }
    if (vtok == 0) {
#pragma unroll
        for (int r = 0; r < GT; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e) sO[wave][r][vpart * VEC + e] = acc[r][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < GT; ++r) {
            sM[wave][r] = m[r];
            sL[wave][r] = l[r];
        }
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
        const int r = idx / D, d = idx - (idx / D) * D;
        if (r >= G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sM[w][r]);
        float o = 0.f, lsum = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = fast_exp2(sM[w][r] - M);
                o = fmaf(sc, sO[w][r][d], o);
                lsum = fmaf(sc, sL[w][r], lsum);
            }
        }
        if (S == 1) {
            const float res = lsum > 0.f ? o / lsum : 0.f;
            const int64_t oi = ((int64_t)row * p.q_heads + (int64_t)g * G + r) * D + d;
            if constexpr (C::kBF16) {
                ((uint16_t*)p.out)[oi] = (uint16_t)f32_to_bf16_bits(res);
            } else {
                ((float*)p.out)[oi] = res;
            }
        } else {
            const int64_t wi = ((int64_t)u * Hkv + g) * S + split;
            p.ws_o[(wi * GT + r) * D + d] = o;
            if (d == 0) {
                p.ws_ml[(wi * GT + r) * 2 + 0] = M;
                p.ws_ml[(wi * GT + r) * 2 + 1] = lsum;
            }
        }
    }
}

// Merge of the split partials of one (unit, kv head).
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void attn_vec_combine_kernel(AttnParams p) {
    const int32_t g = blockIdx.x;
    const int32_t u = blockIdx.y;
    const UnitInfo ui = load_unit(p, u);
    if (ui.q_len != 1) return;
    const int32_t row = ui.q_start;
    if (row < 0 || row >= p.total_q) return;
    const int32_t G = p.group, S = p.num_splits;
    const int64_t w0 = ((int64_t)u * p.kv_heads + g) * S;
    for (int idx = threadIdx.x; idx < GT * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - (idx / D) * D;
        if (r >= G) continue;
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) M = fmaxf(M, p.ws_ml[((w0 + s) * GT + r) * 2]);
        float o = 0.f, lsum = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < S; ++s) {
                const float ms = p.ws_ml[((w0 + s) * GT + r) * 2];
                if (ms == -INFINITY) continue;           // empty split: its o/l are not read
                const float sc = fast_exp2(ms - M);
                o = fmaf(sc, p.ws_o[((w0 + s) * GT + r) * D + d], o);
                lsum = fmaf(sc, p.ws_ml[((w0 + s) * GT + r) * 2 + 1], lsum);
            }
        }
        const float res = lsum > 0.f ? o / lsum : 0.f;
        const int64_t oi = ((int64_t)row * p.q_heads + (int64_t)g * G + r) * D + d;
        if constexpr (sizeof(T) == 2) {
            ((uint16_t*)p.out)[oi] = (uint16_t)f32_to_bf16_bits(res);
        } else {
            ((float*)p.out)[oi] = res;
        }
    }
}

// Zero the output rows that no unit covers.
__global__ __launch_bounds__(256) void zero_uncovered_kernel(AttnParams p, int32_t row_bytes) {
    const int32_t r = blockIdx.x;
    bool covered = false;
    for (int32_t u = 0; u < p.num_units && !covered; ++u) {
        int32_t q0, L;
        if (p.mode == kColumn) {
            q0 = p.seq_info[4 * u];
            L = p.seq_info[4 * u + 1];
        } else if (p.mode == kPagedVarlen) {
            q0 = p.cu_seqlens_q[u];
            L = p.cu_seqlens_q[u + 1] - q0;
        } else {
            q0 = u;
            L = 1;
        }
        if (L > p.max_seqlen_q) L = p.max_seqlen_q;
        covered = (r >= q0) && (L > 0) && (r - q0 < L);
    }
    if (covered) return;
    uint8_t* o = (uint8_t*)p.out + (int64_t)r * row_bytes;
    for (int32_t c = threadIdx.x; c < row_bytes / 16; c += blockDim.x) st16(o + (int64_t)c * 16, u32x4{0u, 0u, 0u, 0u});
}

int32_t vec_group_rows(int32_t group) {
    return group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8;
}

bool attn_vec_supported(pkv_dtype dtype, int32_t head_dim, int32_t group) {
    return (dtype == PKV_F32 || dtype == PKV_BF16) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && group >= 1 && group <= 8;
}

template <typename T, int D, int GT>
static hipError_t launch_vec_t(const AttnParams& p, hipStream_t stream) {
    dim3 grid(p.num_splits, p.kv_heads, p.num_units);
    attn_vec_kernel<T, D, GT><<<grid, dim3(kThreads), 0, stream>>>(p);
    return hipGetLastError();
}

template <typename T, int D, int GT>
static hipError_t launch_combine_t(const AttnParams& p, hipStream_t stream) {
    dim3 grid(p.kv_heads, p.num_units);
    attn_vec_combine_kernel<T, D, GT><<<grid, dim3(256), 0, stream>>>(p);
    return hipGetLastError();
}

#define PKV_DISPATCH(LAUNCH, dtype, head_dim, group, ...)                                   \
    do {                                                                                     \
        const int32_t gt_ = vec_group_rows(group);                                           \
        if (dtype == PKV_BF16) {                                                             \
            if (head_dim == 64) {                                                            \
                if (gt_ == 1) return LAUNCH<__bf16, 64, 1>(__VA_ARGS__);                     \
                if (gt_ == 2) return LAUNCH<__bf16, 64, 2>(__VA_ARGS__);                     \
                if (gt_ == 4) return LAUNCH<__bf16, 64, 4>(__VA_ARGS__);                     \
                return LAUNCH<__bf16, 64, 8>(__VA_ARGS__);                                   \
            } else if (head_dim == 128) {                                                    \
                if (gt_ == 1) return LAUNCH<__bf16, 128, 1>(__VA_ARGS__);                    \
                if (gt_ == 2) return LAUNCH<__bf16, 128, 2>(__VA_ARGS__);                    \
                if (gt_ == 4) return LAUNCH<__bf16, 128, 4>(__VA_ARGS__);                    \
                return LAUNCH<__bf16, 128, 8>(__VA_ARGS__);                                  \
            } else {                                                                         \
                if (gt_ == 1) return LAUNCH<__bf16, 256, 1>(__VA_ARGS__);                    \
                if (gt_ == 2) return LAUNCH<__bf16, 256, 2>(__VA_ARGS__);                    \
                if (gt_ == 4) return LAUNCH<__bf16, 256, 4>(__VA_ARGS__);                    \
                return LAUNCH<__bf16, 256, 8>(__VA_ARGS__);                                  \
            }                                                                                \
        } else {                                                                             \
            if (head_dim == 64) {                                                            \
                if (gt_ == 1) return LAUNCH<float, 64, 1>(__VA_ARGS__);                      \
                if (gt_ == 2) return LAUNCH<float, 64, 2>(__VA_ARGS__);                      \
                if (gt_ == 4) return LAUNCH<float, 64, 4>(__VA_ARGS__);                      \
                return LAUNCH<float, 64, 8>(__VA_ARGS__);                                    \
            } else if (head_dim == 128) {                                                    \
                if (gt_ == 1) return LAUNCH<float, 128, 1>(__VA_ARGS__);                     \
                if (gt_ == 2) return LAUNCH<float, 128, 2>(__VA_ARGS__);                     \
                if (gt_ == 4) return LAUNCH<float, 128, 4>(__VA_ARGS__);                     \
                return LAUNCH<float, 128, 8>(__VA_ARGS__);                                   \
            } else {                                                                         \
                if (gt_ == 1) return LAUNCH<float, 256, 1>(__VA_ARGS__);                     \
                if (gt_ == 2) return LAUNCH<float, 256, 2>(__VA_ARGS__);                     \
                if (gt_ == 4) return LAUNCH<float, 256, 4>(__VA_ARGS__);                     \
                return LAUNCH<float, 256, 8>(__VA_ARGS__);                                   \
            }                                                                                \
        }                                                                                    \
    } while (0)

hipError_t launch_attn_vec(const AttnParams& p, pkv_dtype dtype, int32_t head_dim, hipStream_t stream) {
    if (!attn_vec_supported(dtype, head_dim, p.group)) return hipErrorInvalidValue;
    PKV_DISPATCH(launch_vec_t, dtype, head_dim, p.group, p, stream);
}

hipError_t launch_attn_vec_combine(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                                   hipStream_t stream) {
    if (!attn_vec_supported(dtype, head_dim, p.group)) return hipErrorInvalidValue;
    PKV_DISPATCH(launch_combine_t, dtype, head_dim, p.group, p, stream);
}

hipError_t launch_zero_uncovered(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                                 hipStream_t stream) {
    const int32_t row_bytes = p.q_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4);
    if (p.total_q <= 0) return hipSuccess;
    zero_uncovered_kernel<<<dim3(p.total_q), dim3(256), 0, stream>>>(p, row_bytes);
    return hipGetLastError();
}

}  // namespace pkv
