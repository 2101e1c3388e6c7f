// Matrix-core (MFMA) attention for units with several query rows: chunked
// prefill segments and draft-verify blocks, and any unit whose GQA group is
// larger than the vector path holds.
//
// What it computes (ExecuTorch PR #24073, sdpa_varlen: causal and non-causal
// query blocks over a column store or, with the same arithmetic, a paged cache;
// the causal offset of tiny-llm kv_cache.py causal_kwargs: row i of L new
// queries over E keys sits at position E - L + i): for every query row of the
// unit and each q head of kv head g, softmax(q . K^T * scale) V over that row's
// visible keys.
//
// GQA packing: the unit's L positions times the G heads of one kv head form
// M = L*G rows (row m: position m / G, head m % G), so every K/V element staged
// for a kv head is used by all of its query heads.  A work group (NW waves)
// takes BM = 16*NW of those rows and a range of 64-key chunks.
//
// Per chunk the work group stages K row-major and V transposed ([d][key]) in
// LDS -- keys outside the rows' union of visible ranges, or without storage,
// are staged as zeros -- and each wave runs two bf16 MFMA passes for its 16
// rows with v_mfma_f32_16x16x32_bf16:
//   S^T[key][row] = K . Q^T     (A = K from LDS, B = Q^T from registers)
//   O^T[d][row]  += V^T . P^T   (A = V^T from LDS, B = P^T straight from the
//                                C layout of S^T)
// Working transposed puts one query row per lane column, so the online-softmax
// statistics and the rescale of O stay inside the lane (plus a 4-lane-group
// max/sum).  The k order of the second product is the key permutation the
// first product's C layout leaves in each lane ({4q..4q+3, 16+4q..16+4q+3} for
// lane group q), applied to both operands.
//
// Probabilities are rounded to bf16 for the MFMA and the row sums use the same
// rounded values.  Split-K partials are merged, as in the vector path, by the
// last work group to draw a ticket.
#include "internal.h"
#include "device_util.h"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kIdWindow = 1024;   // block ids staged in LDS at a time

template <int D, int NW, int BN>
struct MfmaCfg {
    static constexpr int NT = 64 * NW;            // threads
    static constexpr int BM = 16 * NW;            // query rows per work group
    static constexpr int KST = D * 2 + 16;        // LDS bytes per staged K row
    static constexpr int VST = BN * 2 + 16;       // LDS bytes per staged V^T row
    static constexpr int DP = D / 8;              // 16-byte parts per key row
    static constexpr int KITEMS = BN * DP;        // K chunk: 16-byte items
    static constexpr int VITEMS = (BN / 2) * DP;  // V chunk: key-pair items
    static constexpr int KPT = (KITEMS + NT - 1) / NT;
    static constexpr int VPT = (VITEMS + NT - 1) / NT;
    static constexpr int KT = BN / 16;            // 16-key tiles per chunk
    static constexpr int KS = D / 32;             // k-steps of the QK product
    static constexpr int DT = D / 16;             // 16-wide d tiles of O
    // V^T rows hold BN/2 key pairs (one dword each).  The pair column is
    // XOR-swizzled by the row's 8-row group (an even amount, so the two pairs a
    // PV operand reads stay adjacent): staging writes from lanes 8 rows apart
    // then land in different banks.
    static constexpr int SWZ_MASK = (BN / 2 - 1) & ~1;
    __device__ static int vcol(int d, int pair) { return pair ^ ((2 * (d >> 3)) & SWZ_MASK); }
    static_assert(KITEMS % NT == 0 && VITEMS % NT == 0, "chunk must split evenly over threads");
    static_assert(BN % 32 == 0, "PV k-steps take 32 keys");
};

template <int D, int NW, int BN, bool PAGED>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(AttnParams p) {
    using C = MfmaCfg<D, NW, BN>;
    constexpr int NT = C::NT, BM = C::BM, KST = C::KST, VST = C::VST, DP = C::DP, KPT = C::KPT,
                  VPT = C::VPT, KT = C::KT, KS = C::KS, DT = C::DT;

    __shared__ __attribute__((aligned(16))) uint8_t sK[BN * KST];
    __shared__ __attribute__((aligned(16))) uint8_t sV[D * VST];
    __shared__ int32_t sIds[kIdWindow];
    __shared__ int32_t sLast;

    const int32_t T = p.mfma_tiles;               // row tiles per (unit, kv head)
    const int32_t S = p.mfma_splits;
    const int32_t tile = blockIdx.x / S;
    const int32_t split = blockIdx.x - tile * S;
    const int32_t g = blockIdx.y;
    const int32_t u = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int lr = lane & 15;                     // this lane's query row within the wave
    const int lq = lane >> 4;                     // lane group 0..3

    const UnitInfo ui = load_unit(p, u);
    const int32_t G = p.group;
    const int32_t L = ui.q_len;
    // Units with one row and a small group belong to the vector path.
    if (L <= 0 || (L == 1 && G <= 8)) return;
    const int32_t Lr = L < p.max_seqlen_q ? L : p.max_seqlen_q;   // rows past the bound: uncovered
    const int32_t M = Lr * G;
    const int32_t m0 = tile * BM;
    if (m0 >= M) return;
    const int32_t E = ui.keys_ok ? ui.kv_end : 0;
    const int32_t Hkv = p.kv_heads;

    // Visible range of position i (row i of the unit).
    auto lo_of = [&](int32_t i) -> int32_t {
        if (p.window <= 0) return 0;
        const int32_t pos = E - L + i;
        const int32_t lo = pos - p.window + 1;
        return lo > 0 ? lo : 0;
    };
    auto hi_of = [&](int32_t i) -> int32_t {
        if (!p.causal) return E;
        const int32_t pos1 = E - L + i + 1;
        return pos1 < E ? (pos1 > 0 ? pos1 : 0) : E;
    };
    const int32_t m_last = min(M, m0 + BM) - 1;
    const int32_t i_first = m0 / G, i_last = m_last / G;
    const int32_t key_lo = lo_of(i_first);                  // the union over this tile's rows
    const int32_t key_hi = max(hi_of(i_last), key_lo);
    const int32_t c_base = (key_lo >> 4) << 4;
    const int32_t nchunk = key_hi > c_base ? (key_hi - c_base + BN - 1) / BN : 0;
    const int32_t cps = (nchunk + S - 1) / S;
    const int32_t c_first = split * cps;
    const int32_t c_end = min(nchunk, c_first + cps);

    // This lane's row.
    const int32_t my_m = m0 + wave * 16 + lr;
    const bool row_ok = my_m < M;
    const int32_t my_i = row_ok ? my_m / G : 0;
    const int32_t my_h = row_ok ? my_m - my_i * G : 0;
    const int32_t my_lo = lo_of(my_i), my_hi = row_ok ? hi_of(my_i) : 0;

    const bool in_rows = row_ok && (ui.q_start + my_i) >= 0 && (ui.q_start + my_i) < p.total_q;

    // Q^T operand: row my_m, d = ks*32 + 8*lq .. +7.
    u32x4 qf[KS];
    {
        const uint8_t* qb = (const uint8_t*)p.q +
                            (((int64_t)(ui.q_start + my_i) * p.q_heads + (int64_t)g * G + my_h) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = in_rows ? ld16(qb + (ks * 32 + 8 * lq) * 2) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x4_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const uint8_t* __restrict__ Kg = (const uint8_t*)p.k;
    const uint8_t* __restrict__ Vg = (const uint8_t*)p.v;
    const int64_t tok_stride = (int64_t)Hkv * D * 2;
    const int64_t head_off = (int64_t)g * D * 2;
    int32_t id_base = -kIdWindow;                 // first block of the staged id window

    // Byte offset of key j (head g) in K or V, or -1 when it has no storage.
    auto key_addr = [&](int32_t j) -> int64_t {
        if constexpr (PAGED) {
            const int32_t id = sIds[(j >> 4) - id_base];
            if (id < 0 || id >= p.num_blocks) return -1;
            return ((int64_t)id * 16 + (j & 15)) * tok_stride + head_off;
        } else {
            int32_t r = j % p.rows;
            return ((int64_t)r * p.cols + ui.col) * tok_stride + head_off;
        }
    };

    // Registers carrying the next chunk from global memory to LDS.
    u32x4 kreg[KPT], vreg[VPT][2];
    auto fetch = [&](int32_t c) {
        const int32_t c0 = c_base + c * BN;
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int ci = tid + k * NT;
            const int kk = ci / DP, part = ci - (ci / DP) * DP;
            const int32_t j = c0 + kk;
            int64_t a = (j >= key_lo && j < key_hi) ? key_addr(j) : -1;
            kreg[k] = a >= 0 ? ld16(Kg + a + part * 16) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vi = tid + k * NT;
            const int kp = vi / DP, part = vi - (vi / DP) * DP;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int32_t j = c0 + 2 * kp + h;
                int64_t a = (j >= key_lo && j < key_hi) ? key_addr(j) : -1;
                vreg[k][h] = a >= 0 ? ld16(Vg + a + part * 16) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            const int ci = tid + k * NT;
            const int kk = ci / DP, part = ci - (ci / DP) * DP;
            st16(sK + kk * KST + part * 16, kreg[k]);
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int vi = tid + k * NT;
            const int kp = vi / DP, part = vi - (vi / DP) * DP;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = word(vreg[k][0], w), b = word(vreg[k][1], w);
                const int d = part * 8 + 2 * w;
                *reinterpret_cast<uint32_t*>(sV + d * VST + C::vcol(d, kp) * 4) = pair_lo(a, b);
                *reinterpret_cast<uint32_t*>(sV + (d + 1) * VST + C::vcol(d + 1, kp) * 4) = pair_hi(a, b);
            }
        }
    };
    // Stage the block ids of [blk, blk + kIdWindow) (paged): every thread calls it.
    auto stage_ids = [&](int32_t blk) {
        __syncthreads();
        for (int k = tid; k < kIdWindow; k += NT) {
            const int32_t b = blk + k;
            sIds[k] = (b < p.max_blocks && b >= 0) ? p.block_table[(int64_t)u * p.max_blocks + b] : -1;
        }
        id_base = blk;
        __syncthreads();
    };
    auto ensure_ids = [&](int32_t c) {
        if constexpr (PAGED) {
            const int32_t b_lo = (c_base + c * BN) >> 4;
            const int32_t b_hi = (c_base + c * BN + BN - 1) >> 4;
            if (b_lo < id_base || b_hi >= id_base + kIdWindow) stage_ids(b_lo);
        }
    };

    if (c_first < c_end) {
        ensure_ids(c_first);
        fetch(c_first);
    }
    for (int32_t c = c_first; c < c_end; ++c) {
        __syncthreads();                          // previous chunk's LDS reads are done
        stage();
        __syncthreads();
        if (c + 1 < c_end) {
            ensure_ids(c + 1);
            fetch(c + 1);                         // in flight during this chunk's math
        }
        const int32_t c0 = c_base + c * BN;

        // ---- S^T = K . Q^T for this wave's 16 rows and the chunk's BN keys ----
        f32x4_t st[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(sK + (kt * 16 + lr) * KST + (ks * 32 + 8 * lq) * 2);
                st[kt] = mfma16(a, qf[ks], st[kt]);
            }
        }
        // ---- mask, online softmax (row = lr; keys kt*16 + 4*lq + e) ----
        float cmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int32_t j = c0 + kt * 16 + 4 * lq + e;
                const bool vis = j >= my_lo && j < my_hi;
                const float v = vis ? st[kt][e] * p.scale_log2 : -INFINITY;
                st[kt][e] = v;
                cmax = fmaxf(cmax, v);
            }
        cmax = fmaxf(cmax, xor_lanes<16>(cmax));
        cmax = fmaxf(cmax, xor_lanes<32>(cmax));
        const float m_new = fmaxf(m_run, cmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        uint32_t pk[KT][2];                       // probabilities, bf16, 4 keys per tile
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            float pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[e] = round_bf16(fast_exp2(st[kt][e] - m_use));
                psum += pr[e];
            }
            pk[kt][0] = pack_bf16(pr[0], pr[1]);
            pk[kt][1] = pack_bf16(pr[2], pr[3]);
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt][0] *= alpha; o[dt][1] *= alpha; o[dt][2] *= alpha; o[dt][3] *= alpha;
        }
        // ---- O^T += V^T . P^T, 32 keys per step: tiles (2s, 2s+1) ----
#pragma unroll
        for (int s2 = 0; s2 < KT / 2; ++s2) {
            const u32x4 b = u32x4{pk[2 * s2][0], pk[2 * s2][1], pk[2 * s2 + 1][0], pk[2 * s2 + 1][1]};
            const int kk0 = s2 * 32 + 4 * lq;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 16 + lr;
                const uint8_t* vrow = sV + d * VST;
                const uint2 lo4 = *reinterpret_cast<const uint2*>(vrow + C::vcol(d, kk0 / 2) * 4);
                const uint2 hi4 = *reinterpret_cast<const uint2*>(vrow + C::vcol(d, (kk0 + 16) / 2) * 4);
                o[dt] = mfma16(u32x4{lo4.x, lo4.y, hi4.x, hi4.y}, b, o[dt]);
            }
        }
    }

    // Row sum across the 4 lane groups.
    l_run += xor_lanes<16>(l_run);
    l_run += xor_lanes<32>(l_run);

    // This lane holds O^T[d][row] for d = dt*16 + 4*lq + e.
    const int64_t orow = ((int64_t)(ui.q_start + my_i) * p.q_heads + (int64_t)g * G + my_h) * D;
    if (S == 1) {
        if (in_rows) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 16 + 4 * lq;
                const uint2 w2 = uint2{pack_bf16(o[dt][0] * inv, o[dt][1] * inv),
                                       pack_bf16(o[dt][2] * inv, o[dt][3] * inv)};
                *reinterpret_cast<uint2*>((uint16_t*)p.out + orow + d) = w2;
            }
        }
        return;
    }

    // ---- split-K partials: [unit, kv head, tile, split][BM][D] and (m, l) ----
    const int64_t wi = (((int64_t)u * Hkv + g) * T + tile) * S + split;
    const int rloc = wave * 16 + lr;
    float* po = p.mws_o + (wi * BM + rloc) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        st_agent2(po + dt * 16 + 4 * lq, o[dt][0], o[dt][1]);
        st_agent2(po + dt * 16 + 4 * lq + 2, o[dt][2], o[dt][3]);
    }
    if (lq == 0) st_agent2(&p.mws_ml[(wi * BM + rloc) * 2], m_run, l_run);
    wait_vm_all();
    __syncthreads();
    int32_t* ticket = p.mws_ticket + (((int64_t)u * Hkv + g) * T + tile) * kTicketStride;
    if (tid == 0)
        sLast = (__hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1);
    __syncthreads();
    if (!sLast) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Merge: each thread takes 4 consecutive outputs of one row, 16 splits in flight.
    const int64_t w0 = (((int64_t)u * Hkv + g) * T + tile) * S;
    constexpr int CH = 16;
    for (int idx = tid; idx < BM * (D / 4); idx += NT) {
        const int r = idx / (D / 4), d4 = (idx - r * (D / 4)) * 4;
        const int32_t mm = m0 + r;
        if (mm >= M) continue;
        const int32_t ii = mm / G, hh = mm - (mm / G) * G;
        if (ui.q_start + ii < 0 || ui.q_start + ii >= p.total_q) continue;
        const float* osrc = p.mws_o + (w0 * BM + r) * D + d4;
        const float* msrc = p.mws_ml + (w0 * BM + r) * 2;
        const int64_t ostride = (int64_t)BM * D, mstride = (int64_t)BM * 2;
        float Mx = -INFINITY, tot = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < S; s0 += CH) {
            float2 ml[CH];
            float4 x[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const int sk = min(s0 + k, S - 1);
                ml[k] = *reinterpret_cast<const float2*>(msrc + sk * mstride);
                x[k] = *reinterpret_cast<const float4*>(osrc + sk * ostride);
            }
            // No branch on loaded values, so all loads of a pass are in flight together.
            float Mc = Mx;
#pragma unroll
            for (int k = 0; k < CH; ++k) Mc = (s0 + k < S) ? fmaxf(Mc, ml[k].x) : Mc;
            const float Mu = (Mc == -INFINITY) ? 0.f : Mc;
            const float a = fast_exp2(Mx - Mu);     // 0 while nothing was visible
            tot *= a;
            acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const float w = (s0 + k < S) ? fast_exp2(ml[k].x - Mu) : 0.f;
                tot = fmaf(w, ml[k].y, tot);
                acc.x = fmaf(w, x[k].x, acc.x);
                acc.y = fmaf(w, x[k].y, acc.y);
                acc.z = fmaf(w, x[k].z, acc.z);
                acc.w = fmaf(w, x[k].w, acc.w);
            }
            Mx = Mc;
        }
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        const int64_t oi = ((int64_t)(ui.q_start + ii) * p.q_heads + (int64_t)g * G + hh) * D + d4;
        const uint2 w2 = uint2{pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv)};
        *reinterpret_cast<uint2*>((uint16_t*)p.out + oi) = w2;
    }
}

int32_t mfma_rows_per_group(int32_t head_dim) { return head_dim == 64 ? 16 * 4 : 16 * 8; }
int32_t mfma_chunk_keys(int32_t head_dim) { return head_dim == 256 ? 32 : 64; }

bool attn_mfma_supported(pkv_dtype dtype, int32_t head_dim) {
    return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

template <int D, int NW, int BN>
static hipError_t launch_mfma_t(const AttnParams& p, hipStream_t stream) {
    dim3 grid(p.mfma_tiles * p.mfma_splits, p.kv_heads, p.num_units);
    if (p.mode == kColumn) {
        attn_mfma_kernel<D, NW, BN, false><<<grid, dim3(64 * NW), 0, stream>>>(p);
    } else {
        attn_mfma_kernel<D, NW, BN, true><<<grid, dim3(64 * NW), 0, stream>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams& p, pkv_dtype dtype, int32_t head_dim, hipStream_t stream) {
    if (!attn_mfma_supported(dtype, head_dim)) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_mfma_t<64, 4, 64>(p, stream);
    if (head_dim == 128) return launch_mfma_t<128, 8, 64>(p, stream);
    return launch_mfma_t<256, 8, 32>(p, stream);
}

}  // namespace pkv
