// Vector-ALU decode attention: units with one query row, GQA group <= 8.
//
// What it computes (vLLM-Omni paged_decode, PagedDecodeCache.attend calling
// flash_attn_varlen_func with max_seqlen_q = 1; ExecuTorch PR #24073 for
// sdpa_varlen's column store, window, zeroed rows and split-K): for the query
// row of a unit and each q head h of kv head g, softmax(q_h . K^T * scale) V
// over the unit's visible live keys, read through the block table or ring.
// With k_new/v_new (paged decode) the same kernel also writes this step's K/V
// to position E-1 and attends over it as part of the prefix, as
// PagedDecodeCache.attend does (append, then attend).
//
// One kernel per call.  Work decomposition: one work group (4 waves) per
// (split, kv head, unit).  The unit's visible keys, as whole 16-token blocks,
// are cut into `splits` contiguous block ranges of the live range, so the work
// per call follows the live length, not the bucket.  Wave w of a work
// group takes blocks w, w+4, ... of its range: the reduction order depends only
// on logical positions, so a permuted block table gives bit-identical results.
// Each wave gathers the block ids of all its blocks with one vector load and
// keeps the next block's K/V loads in flight while it computes the current one.
//
// Per block a wave holds the 16 tokens' K for its kv head in registers laid
// out KLPT lanes per token (q . k needs only a KLPT-lane DPP reduction) and
// their V one 16-byte chunk per lane.  All G query heads of the group are
// scored against the same registers (GQA sharing).  Scores go through an
// online softmax (running max per head, wave-uniform after a cross-lane max);
// probabilities move from the K layout to the V layout through a per-wave LDS
// slab.  bf16 uses v_dot2_f32_bf16 for both products, with probabilities
// rounded to bf16 (the running sum uses the same rounded values, so a constant
// V comes back exactly); fp32 uses fma.  Accumulation is fp32.
//
// Split-K: each work group leaves (o, m, l) partials; the last work group of a
// (unit, kv head) to arrive -- an atomic ticket, reset by that work group --
// merges them with a log-sum-exp weighting and writes the output.
//
// Keys outside the visible range never reach the sums: their scores become
// -inf by selection and their V chunks are replaced by 0, so NaN or Inf
// garbage in storage past seqused_k cannot leak.
#include "internal.h"
#include "device_util.h"

namespace pkv {

constexpr int kWaves = 4;
// Slack of the softmax reference point, in log2 units (probabilities < 256).
constexpr float kLazyLog2 = 8.f;
constexpr int kThreads = 64 * kWaves;

template <typename T, int D, int GT>
struct VecCfg {
    static constexpr bool kBF16 = sizeof(T) == 2;
    static constexpr int EB = sizeof(T);
    static constexpr int VEC = 16 / EB;       // elements per 16-byte chunk
    static constexpr int RC = D / VEC;        // chunks per token row of one head
    static constexpr int qdw(int klpt) { return GT * (RC / klpt) * 4; }
    // Lanes per token in the K layout: the fewest that keep q in <= 64 dwords,
    // but at least 8 where a row has 8 chunks, so that one load instruction
    // covers whole 128-byte lines of its tokens (with 4 lanes per token each
    // line was requested by two instructions, half a line each: the batched
    // 64-sequence decode streamed about 10 % slower).
    static constexpr int KLPT = (RC >= 8 && qdw(8) <= 64) ? 8
                              : (RC >= 4 && RC < 8 && qdw(4) <= 64) ? 4
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
    // V-layout token groups kept apart in LDS for the final merge (<= 32 KiB).
    static constexpr int vr_fit(int vr) { return 4 * vr * GT * D * 4 <= 32768 || vr == 1 ? vr : vr_fit(vr / 2); }
    static constexpr int VR = vr_fit(VTPW);
};

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
    if constexpr (sizeof(T) == 2) {
        ((uint16_t*)out)[idx] = (uint16_t)f32_to_bf16_bits(v);
    } else {
        ((float*)out)[idx] = v;
    }
}

// The vector path's work item w.  Normally a unit.  In row mode (fp32 calls
// with several query rows per unit) item w is row i = w % max_seqlen_q of unit
// w / max_seqlen_q, seen as a single query: q_start moves to that row and
// q_len becomes L - i, so that its position E - q_len is the row's E - L + i;
// a row past the unit's rows (or past max_seqlen_q) gets q_len 0.  `tab` is
// the unit whose block-table row or column the keys come from.
struct VecItem {
    UnitInfo ui;
    int32_t tab;
};
__device__ __forceinline__ VecItem load_vec_item(const AttnParams& p, int32_t w) {
    VecItem it;
    if (!p.row_mode) {
        it.tab = w;
        it.ui = load_unit(p, w);
        return it;
    }
    const int32_t R = p.max_seqlen_q;
    it.tab = w / R;
    const int32_t i = w - it.tab * R;
    it.ui = load_unit(p, it.tab);
    const int32_t L = it.ui.q_len < R ? it.ui.q_len : R;
    if (i >= L) {
        it.ui.q_len = 0;
    } else {
        it.ui.q_start += i;
        it.ui.q_len -= i;
    }
    return it;
}

// Whether the vector path computes an item: a unit of one query row, the first
// row of any unit when the call's static bound max_seqlen_q is 1 (the
// matrix-core path takes the other multi-row units), or any covered row in
// row mode.
__device__ __forceinline__ bool vec_takes(const AttnParams& p, const UnitInfo& ui) {
    return ui.q_len == 1 || (ui.q_len > 1 && (p.max_seqlen_q == 1 || p.row_mode));
}

// Live 16-key blocks of unit u for the vector path, or -1 when the unit is
// not this path's (see vec_takes, or its row outside the output).
__device__ __forceinline__ int32_t vec_unit_blocks(const AttnParams& p, int32_t u) {
    const UnitInfo ui = load_vec_item(p, u).ui;
    if (!vec_takes(p, ui) || ui.q_start < 0 || ui.q_start >= p.total_q) return -1;
    const int32_t E = ui.keys_ok ? ui.kv_end : 0;
    const KeyRange kr = first_row_keys(p, E, ui.q_len, ui.pad);
    const int32_t b_end = (kr.hi + 15) >> 4, b_first = kr.lo >> 4;
    return b_end > b_first ? b_end - b_first : 0;
}


// Log-sum-exp merge of this lane's (M, tot, o) with lane (lane ^ ST)'s.
template <int ST>
__device__ __forceinline__ void combine_lanes(float& M, float& tot, float4& o) {
    const float Mo = xor_lanes<ST>(M), to = xor_lanes<ST>(tot);
    const float ox = xor_lanes<ST>(o.x), oy = xor_lanes<ST>(o.y);
    const float oz = xor_lanes<ST>(o.z), ow = xor_lanes<ST>(o.w);
    const float Mn = fmaxf(M, Mo);
    const float Mu = (Mn == -INFINITY) ? 0.f : Mn;
    const float a = fast_exp2(M - Mu), b = fast_exp2(Mo - Mu);
    tot = fmaf(a, tot, b * to);
    o.x = fmaf(a, o.x, b * ox);
    o.y = fmaf(a, o.y, b * oy);
    o.z = fmaf(a, o.z, b * oz);
    o.w = fmaf(a, o.w, b * ow);
    M = Mn;
}

// Merge of the S split partials of one (unit, kv head).  NP consecutive lanes
// share one group of 4 outputs of one head; lane part k of the group takes the
// splits k, k + NP, ...  Every load of a pass is issued before any is used and
// nothing branches on loaded values, so a pass costs one memory round trip.
// Splits past S are clamped to S-1 and weighted 0; an empty split (m = -inf)
// gets weight 0.  The NP lane results meet through lane swizzles.
template <typename T, int D, int GT>
__device__ __forceinline__ void merge_splits(const AttnParams& p, int32_t g, int32_t row, int32_t slot0,
                                             int32_t S) {
    constexpr int ITEMS = GT * (D / 4);
    constexpr int NP = ITEMS >= kThreads ? 1 : (kThreads / ITEMS > 16 ? 16 : kThreads / ITEMS);
    constexpr int CH = NP == 1 ? 32 : NP == 2 ? 16 : 8;
    const int32_t G = p.group, Hkv = p.kv_heads;
    const int64_t w0 = (int64_t)slot0 * Hkv + g;
    const int part = threadIdx.x % NP;
    for (int item = threadIdx.x / NP; item < ITEMS; item += kThreads / NP) {
        const int r = item / (D / 4), d4 = (item - r * (D / 4)) * 4;
        if (r >= G) continue;                   // uniform over the NP lanes of an item
        const float* osrc = p.ws_o + (w0 * GT + r) * D + d4;
        const float* msrc = p.ws_ml + (w0 * GT + r) * 2;
        const int64_t ostride = (int64_t)Hkv * GT * D, mstride = (int64_t)Hkv * GT * 2;
        float M = -INFINITY, tot = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < S; s0 += NP * CH) {
            float2 ml[CH];
            float4 x[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const int sk = min(s0 + part + NP * k, S - 1);
                ml[k] = *reinterpret_cast<const float2*>(msrc + sk * mstride);
                x[k] = *reinterpret_cast<const float4*>(osrc + sk * ostride);
            }
            float Mc = M;
#pragma unroll
            for (int k = 0; k < CH; ++k) Mc = (s0 + part + NP * k < S) ? fmaxf(Mc, ml[k].x) : Mc;
            const float Mu = (Mc == -INFINITY) ? 0.f : Mc;
            const float a = fast_exp2(M - Mu);  // 0 while nothing was visible
            tot *= a;
            o.x *= a; o.y *= a; o.z *= a; o.w *= a;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const float w = (s0 + part + NP * k < S) ? fast_exp2(ml[k].x - Mu) : 0.f;
                tot = fmaf(w, ml[k].y, tot);
                o.x = fmaf(w, x[k].x, o.x);
                o.y = fmaf(w, x[k].y, o.y);
                o.z = fmaf(w, x[k].z, o.z);
                o.w = fmaf(w, x[k].w, o.w);
            }
            M = Mc;
        }
        if constexpr (NP > 1) combine_lanes<1>(M, tot, o);
        if constexpr (NP > 2) combine_lanes<2>(M, tot, o);
        if constexpr (NP > 4) combine_lanes<4>(M, tot, o);
        if constexpr (NP > 8) combine_lanes<8>(M, tot, o);
        if (part != 0) continue;
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        const int64_t oi = ((int64_t)row * p.q_heads + (int64_t)g * G + r) * D + d4;
        store_out<T>(p.out, oi + 0, o.x * inv);
        store_out<T>(p.out, oi + 1, o.y * inv);
        store_out<T>(p.out, oi + 2, o.z * inv);
        store_out<T>(p.out, oi + 3, o.w * inv);
    }
}

// Waves per SIMD the register budget is held to: two (at most 256 VGPRs) for
// the shapes that fit -- the pipelined block loop otherwise grows past that
// and halves occupancy -- one for the large ones (head_dim 256, a group of 8,
// fp32 above head_dim 64), which spill when held to 256.
template <typename T, int D, int GT>
constexpr int vec_waves_per_simd() {
    return (sizeof(T) == 2 ? (D <= 128 && GT <= 4) : (D <= 64 && GT <= 4)) ? 2 : 1;
}

template <typename T, int D, int GT, bool PAGED>
__global__ __launch_bounds__(kThreads, (vec_waves_per_simd<T, D, GT>())) void attn_vec_kernel(AttnParams p) {
    using C = VecCfg<T, D, GT>;
    constexpr int EB = C::EB, VEC = C::VEC, KLPT = C::KLPT, KCH = C::KCH, KTPW = C::KTPW,
                  KNI = C::KNI, VLPT = C::VLPT, VTPW = C::VTPW, VNI = C::VNI;

    __shared__ float sP[kWaves][16 * GT];
    __shared__ float sAcc[kWaves][C::VR][GT][D];
    __shared__ float sLv[kWaves][C::VR][GT];
    __shared__ float sM[kWaves][GT];
    __shared__ int sLast;
    __shared__ int32_t sWork[4];

    // The kv head is the fastest grid dimension: the work groups reading the
    // heads of the same blocks run together and share DRAM rows.  Those of kv
    // head 0 also zero their share of the rows no unit covers.
    const int32_t g = blockIdx.x;
    if (p.zero_rows && g == 0) {
        __shared__ uint32_t sTodo;
        zero_rows_share(p, p.q_heads * D * (int32_t)sizeof(T), &sTodo, kThreads);
    }
    const int32_t slot = blockIdx.y;
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int kpart = lane % KLPT, ktok = lane / KLPT;
    const int vpart = lane % VLPT, vtok = lane / VLPT;

    // Which unit and split this work group takes (slot = blockIdx.y):
    //  - one unit: split = slot of num_splits;
    //  - one split per unit: unit = slot;
    //  - otherwise the num_splits * units slots are dealt over the units: a
    //    unit of nb live blocks gets max(1, ceil(nb / c)) consecutive slots (at
    //    least one, so an empty unit still writes its zero row), c the smallest
    //    block count per slot for which the deal fits the slots.
    int32_t u, split, S, slot0;
    if (p.vec_units == 1) {
        u = 0; split = slot; S = p.num_splits; slot0 = 0;
    } else if (p.num_splits == 1) {
        u = slot; split = 0; S = 1; slot0 = u;
    } else {
        if (wave == 0) {
            const int32_t U = p.vec_units;
            const int64_t W = (int64_t)p.num_splits * U;
            const int32_t per = (U + 63) / 64;
            const int32_t ub = lane * per, ue = min(U, ub + per);
            auto unit_n = [&](int32_t uu) { return vec_unit_blocks(p, uu); };
            const DealItems items = deal_items(unit_n, ub, ue);
            const int32_t c = deal_size(items, unit_n, W);
            int32_t cnt = 0;
            deal_for_each(items, unit_n, [&](int32_t, int32_t n) { cnt += deal_slots_of(n, c); });
            int32_t incl = cnt;
#pragma unroll
            for (int st = 1; st < 64; st *= 2) {
                const int32_t y = __shfl_up(incl, st, 64);
                if (lane >= st) incl += y;
            }
            if (lane == 0) sWork[0] = -1;
            int32_t acc = incl - cnt;
            const int32_t w = slot;
            deal_for_each(items, unit_n, [&](int32_t uu, int32_t nb) {
                const int32_t n = deal_slots_of(nb, c);
                if (w >= acc && w < acc + n) {
                    sWork[0] = uu; sWork[1] = w - acc; sWork[2] = n; sWork[3] = acc;
                }
                acc += n;
            });
        }
        __syncthreads();
        u = sWork[0]; split = sWork[1]; S = sWork[2]; slot0 = sWork[3];
        if (u < 0) return;                          // a spare slot
    }

    const VecItem item = load_vec_item(p, u);
    const UnitInfo& ui = item.ui;
    const int64_t tab_row = (int64_t)item.tab * p.max_blocks;   // block-table row (paged)
    if (!vec_takes(p, ui)) return;                  // other units are not this path's
    const int32_t row = ui.q_start;
    if (row < 0 || row >= p.total_q) return;

    const int32_t G = p.group;
    const int32_t Hkv = p.kv_heads;
    const int32_t E = ui.keys_ok ? ui.kv_end : 0;
    // One query row at position E - q_len: keys [lo, hi) with the causal,
    // window and left-padding bounds.
    const KeyRange krange = first_row_keys(p, E, ui.q_len, ui.pad);
    const int32_t lo = krange.lo;
    const int32_t hi = krange.hi;
    const int32_t b_end = (hi + 15) >> 4;
    const int32_t b_first = lo >> 4;
    const int32_t nblk = b_end > b_first ? b_end - b_first : 0;
    const int32_t bps = (nblk + S - 1) / S;
    const int32_t sb = b_first + split * bps;
    const int32_t se = min(b_end, sb + bps);
    int32_t ids = -1;               // lane i: pool block of this wave's i-th block
    if constexpr (PAGED) {
        const int32_t blk = sb + wave + kWaves * lane;
        if (blk < se) ids = p.block_table[tab_row + blk];
    }
    // Blocks of this wave: first + 4 i, i < nb.
    const int32_t first = sb + wave;
    const int32_t nb = first < se ? (se - first + kWaves - 1) / kWaves : 0;

    const uint8_t* __restrict__ Kb = (const uint8_t*)p.k;
    const uint8_t* __restrict__ Vb = (const uint8_t*)p.v;
    const int64_t tok_stride = (int64_t)Hkv * D * EB;        // bytes between tokens of a block
    const int64_t head_off = (int64_t)g * D * EB;

    // Fused append: token E-1 comes from k_new/v_new and is written to its slot.
    const bool fuse = p.k_new != nullptr && E > 0;
    const int32_t pn = E - 1;
    const uint8_t* kn = fuse ? (const uint8_t*)p.k_new + ((int64_t)u * Hkv + g) * D * EB : nullptr;
    const uint8_t* vn = fuse ? (const uint8_t*)p.v_new + ((int64_t)u * Hkv + g) * D * EB : nullptr;

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

    // m: running max per head (wave-uniform); acc and lv: this lane's share of
    // the output numerator and of the softmax denominator, in the V layout.
    float m[GT], lv[GT], acc[GT][VEC];
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        m[r] = -INFINITY;
        lv[r] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][e] = 0.f;
    }

    // Byte offset of token tt of block `blk` (id: its pool block when paged).
    // Paged: the block's base is uniform and the lane part fits 32 bits.
    const int64_t col_stride = (int64_t)p.cols * tok_stride;    // ring: bytes per store row
    auto tok_addr = [&](int32_t blk, int32_t id, int tt) -> int64_t {
        if constexpr (PAGED) {
            return (int64_t)id * (16 * tok_stride) + head_off + (int32_t)(tt * (int32_t)tok_stride);
        } else {
            int32_t r = (blk * 16) % p.rows + tt;
            if (r >= p.rows) r -= p.rows;
            if (r >= p.rows) r %= p.rows;       // rings shorter than a block
            return (int64_t)r * col_stride + (int64_t)ui.col * tok_stride + head_off;
        }
    };
    auto id_ok = [&](int32_t id) { return !PAGED || (id >= 0 && id < p.num_blocks); };

    // Fused append.  Position E-1 sits in the last live block, which is the
    // last block of the one wave that owns it.  Inside the loop, the lanes of
    // that wave that would read the row from the cache read it from k_new /
    // v_new instead (an address choice, so the block stays in the load
    // pipeline like any other).  No other work group reads that row in this
    // call, so the wave may write it to its slot at either end of the loop:
    // after it where registers are to spare (the store's waits then never
    // delay the first block's loads), before it for the shapes held to one
    // wave per SIMD (whose loop would otherwise carry the store's operands).
    const int32_t pblk = pn >> 4, ptt = pn & 15;
    const bool own_new = fuse && pblk >= sb && pblk < se && (pblk - sb) % kWaves == wave;
    const int32_t pid = (own_new && PAGED) ? p.block_table[tab_row + pblk] : 0;
    constexpr bool kStoreAfter = vec_waves_per_simd<T, D, GT>() == 2;
    auto store_new_row = [&]() {
        if (own_new && id_ok(pid) && lane < D * EB / 16) {
            const int64_t a = tok_addr(pblk, pid, ptt);
            st16((uint8_t*)p.k + a + lane * 16, ld16(kn + lane * 16));
            st16((uint8_t*)p.v + a + lane * 16, ld16(vn + lane * 16));
        }
    };
    if constexpr (!kStoreAfter) store_new_row();

    // Every load of the block loop is issued unconditionally -- a block with
    // no storage loads pool block 0 and is skipped when processed -- so the
    // compiler's wait counts see the same loads on every path and wait only
    // for the block being processed, never for the one in flight behind it.
    auto load = [&](int i, int32_t id, u32x4 (&kr)[KNI][KCH], u32x4 (&vr)[VNI]) {
        const int32_t blk = first + kWaves * i;
        const int32_t idc = id_ok(id) ? id : 0;
        const bool own = own_new && blk == pblk;        // wave-uniform
#pragma unroll
        for (int j = 0; j < KNI; ++j) {
            const int tt = j * KTPW + ktok;
            const uint8_t* src = Kb + tok_addr(blk, idc, tt) + kpart * 16;
            if (own && tt == ptt) src = kn + kpart * 16;
#pragma unroll
            for (int c = 0; c < KCH; ++c) kr[j][c] = ld16_stream(src + KLPT * c * 16);
        }
#pragma unroll
        for (int j = 0; j < VNI; ++j) {
            const int tt = j * VTPW + vtok;
            const uint8_t* src = Vb + tok_addr(blk, idc, tt) + vpart * 16;
            if (own && tt == ptt) src = vn + vpart * 16;
            vr[j] = ld16_stream(src);
        }
    };

    float* P = sP[wave];
    auto process = [&](int i, int32_t id, u32x4 (&kr)[KNI][KCH], u32x4 (&vr)[VNI]) {
        if (!id_ok(id)) return;                 // no storage: these keys contribute nothing
        const int32_t t0 = (first + kWaves * i) * 16;
        const bool full = (t0 >= lo) && (t0 + 16 <= hi);

        // ---- scores for every head of the group (all lanes of a token agree) ----
        float s[KNI][GT];
#pragma unroll
        for (int j = 0; j < KNI; ++j) {
            const int32_t t = t0 + j * KTPW + ktok;
            const bool vis = full || (t >= lo && t < hi);
#pragma unroll
            for (int r = 0; r < GT; ++r) {
                float d = 0.f;
#pragma unroll
                for (int c = 0; c < KCH; ++c) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        if constexpr (C::kBF16) {
                            d = dot2_bf16(word(qr[r][c], w), word(kr[j][c], w), d);
                        } else {
                            d = fmaf(__builtin_bit_cast(float, word(qr[r][c], w)),
                                     __builtin_bit_cast(float, word(kr[j][c], w)), d);
                        }
                    }
                }
                d = group_sum<KLPT>(d) * p.scale_log2;
                s[j][r] = vis ? d : -INFINITY;
            }
        }

        // ---- online softmax: per-head block max, rescale factor, probabilities ----
        float alpha[GT];
        bool rescale = false;
#pragma unroll
        for (int r = 0; r < GT; ++r) {
            float mb = s[0][r];
#pragma unroll
            for (int j = 1; j < KNI; ++j) mb = fmaxf(mb, s[j][r]);
            mb = across_groups<KLPT, true>(mb);
            // The head's reference point moves only when a block's maximum
            // passes it by more than kLazyLog2 (probabilities stay below
            // 2^kLazyLog2), so most blocks skip the rescale.
            const bool bump = mb > m[r] + kLazyLog2;
            const float m_new = bump ? mb : m[r];
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            alpha[r] = bump ? fast_exp2(m[r] - m_use) : 1.f;
            rescale |= bump;
            m[r] = m_new;
#pragma unroll
            for (int j = 0; j < KNI; ++j) {
                float pr = fast_exp2(s[j][r] - m_use);
                if constexpr (C::kBF16) pr = round_bf16(pr);
                s[j][r] = pr;
            }
        }

        // ---- probabilities from the K layout to the V layout through LDS ----
        if (kpart == 0) {
#pragma unroll
            for (int j = 0; j < KNI; ++j)
#pragma unroll
                for (int r = 0; r < GT; ++r) P[(j * KTPW + ktok) * GT + r] = s[j][r];
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);

        if (rescale) {   // wave-uniform: m is identical in every lane
#pragma unroll
            for (int r = 0; r < GT; ++r) {
                lv[r] *= alpha[r];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[r][e] *= alpha[r];
            }
        }
        if (!full) {
#pragma unroll
            for (int j = 0; j < VNI; ++j) {
                const int32_t t = t0 + j * VTPW + vtok;
                if (!(t >= lo && t < hi)) vr[j] = u32x4{0u, 0u, 0u, 0u};
            }
        }

        // ---- PV ----
        if constexpr (C::kBF16) {
#pragma unroll
            for (int j = 0; j < VNI; j += 2) {
                float pa[GT], pb[GT];
#pragma unroll
                for (int r = 0; r < GT; ++r) {
                    pa[r] = P[(j * VTPW + vtok) * GT + r];
                    pb[r] = P[((j + 1) * VTPW + vtok) * GT + r];
                }
                uint32_t vp[VEC];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    vp[2 * w] = pair_lo(word(vr[j], w), word(vr[j + 1], w));
                    vp[2 * w + 1] = pair_hi(word(vr[j], w), word(vr[j + 1], w));
                }
#pragma unroll
                for (int r = 0; r < GT; ++r) {
                    lv[r] += pa[r] + pb[r];
                    const uint32_t pp = pair_hi(__builtin_bit_cast(uint32_t, pa[r]),
                                                __builtin_bit_cast(uint32_t, pb[r]));
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[r][e] = dot2_bf16(pp, vp[e], acc[r][e]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < VNI; ++j) {
#pragma unroll
                for (int r = 0; r < GT; ++r) {
                    const float pr = P[(j * VTPW + vtok) * GT + r];
                    lv[r] += pr;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        acc[r][e] = fmaf(pr, __builtin_bit_cast(float, word(vr[j], e)), acc[r][e]);
                }
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // ---- block loop, next block's loads in flight during the current compute ----
    // Groups of up to 64 blocks per wave: lane l holds the pool id of the
    // group's l-th block (the first group's ids were read above).
    {
        u32x4 ka[KNI][KCH], kb[KNI][KCH], va[VNI], vb[VNI];
        for (int g0 = 0; g0 < nb; g0 += 64) {
            const int gn = min(64, nb - g0);
            if constexpr (PAGED) {
                if (g0 > 0) {
                    const int32_t blk = first + kWaves * (g0 + lane);
                    ids = lane < gn ? p.block_table[tab_row + blk] : -1;
                }
            }
            auto id_of = [&](int k) -> int32_t { return PAGED ? __builtin_amdgcn_readlane(ids, k) : 0; };
            int32_t ida = id_of(0), idb = 0;
            load(g0, ida, ka, va);
            int k = 0;
            for (; k + 2 < gn; k += 2) {
                idb = id_of(k + 1);
                load(g0 + k + 1, idb, kb, vb);
                process(g0 + k, ida, ka, va);
                ida = id_of(k + 2);
                load(g0 + k + 2, ida, ka, va);
                process(g0 + k + 1, idb, kb, vb);
            }
            if (k + 1 < gn) {
                idb = id_of(k + 1);
                load(g0 + k + 1, idb, kb, vb);
                process(g0 + k, ida, ka, va);
                process(g0 + k + 1, idb, kb, vb);
            } else {
                process(g0 + k, ida, ka, va);
            }
        }
    }

    if constexpr (kStoreAfter) store_new_row();

    // ---- merge lanes, then waves, through LDS ----
    // acc and lv: fold the V-layout token groups down to VR groups, park them
    // in LDS; m is wave-uniform.
    constexpr int VR = C::VR;
    auto fold = [&](float x) -> float {
        if constexpr (VR * VLPT < 64) {
#pragma unroll
            for (int st = VR * VLPT; st < 64; st *= 2) {
                if (st == 1) x += xor_lanes<1>(x);
                else if (st == 2) x += xor_lanes<2>(x);
                else if (st == 4) x += xor_lanes<4>(x);
                else if (st == 8) x += xor_lanes<8>(x);
                else if (st == 16) x = swap_op16<false>(x);
                else x = swap_op32<false>(x);
            }
        }
        return x;
    };
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        lv[r] = fold(lv[r]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r][e] = fold(acc[r][e]);
    }
    if (vtok < VR) {
#pragma unroll
        for (int r = 0; r < GT; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e) sAcc[wave][vtok][r][vpart * VEC + e] = acc[r][e];
        if (vpart == 0) {
#pragma unroll
            for (int r = 0; r < GT; ++r) sLv[wave][vtok][r] = lv[r];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < GT; ++r) sM[wave][r] = m[r];
    }
    __syncthreads();

    const int64_t wi = (int64_t)(slot0 + split) * Hkv + g;
    for (int idx = threadIdx.x; idx < GT * (D / 2); idx += kThreads) {
        const int r = idx / (D / 2), d = (idx - r * (D / 2)) * 2;
        if (r >= G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sM[w][r]);
        float o0 = 0.f, o1 = 0.f, lsum = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float sc = fast_exp2(sM[w][r] - M);
                float ow0 = 0.f, ow1 = 0.f, lw = 0.f;
#pragma unroll
                for (int t = 0; t < VR; ++t) {
                    const float2 a2 = *reinterpret_cast<const float2*>(&sAcc[w][t][r][d]);
                    ow0 += a2.x;
                    ow1 += a2.y;
                    lw += sLv[w][t][r];
                }
                o0 = fmaf(sc, ow0, o0);
                o1 = fmaf(sc, ow1, o1);
                lsum = fmaf(sc, lw, lsum);
            }
        }
        if (S == 1) {
            const int64_t oi = ((int64_t)row * p.q_heads + (int64_t)g * G + r) * D + d;
            store_out<T>(p.out, oi, lsum > 0.f ? o0 / lsum : 0.f);
            store_out<T>(p.out, oi + 1, lsum > 0.f ? o1 / lsum : 0.f);
        } else {
            st_agent2(&p.ws_o[(wi * GT + r) * D + d], o0, o1);
            if (d == 0) st_agent2(&p.ws_ml[(wi * GT + r) * 2], M, lsum);
        }
    }
    if (S == 1) return;

    // ---- split-K: the last work group of this (unit, kv head) merges ----
    // Partials go out with device-coherent stores; once every wave's stores
    // have completed, one thread takes a ticket.  The work group drawing the
    // last ticket drops its stale cache lines (an agent-scope acquire: no
    // writeback) and reads all partials with 16-byte loads (one round trip;
    // device-coherent 8-byte loads instead measured slower).
    wait_vm_all();
    __syncthreads();
    int32_t* ticket = p.ws_ticket + ((int64_t)u * Hkv + g) * kTicketStride;
    if (threadIdx.x == 0)
        sLast = (__hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1);
    __syncthreads();
    if (!sLast) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0)                       // ready for the next call
        __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_splits<T, D, GT>(p, g, row, slot0, S);
}

// Zero the output rows that no unit covers, as a launch of its own (calls
// with no unit to attend): kZeroRows rows per work group.
constexpr int kZeroRows = 16;

__global__ __launch_bounds__(256) void zero_uncovered_kernel(AttnParams p, int32_t row_bytes) {
    __shared__ uint32_t sTodo;
    const int32_t r0 = blockIdx.x * kZeroRows;
    const int32_t n = min(kZeroRows, p.total_q - r0);
    zero_uncovered_rows(p, r0, n, row_bytes, &sTodo, 256);
}

int32_t vec_group_rows(int32_t group) {
    return group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8;
}

int32_t vec_slots(int32_t units, int32_t splits) {
    if (units <= 1) return splits;
    if (splits <= 1) return units;
    return splits * units;
}

size_t ticket_bytes(int32_t units, int32_t kv_heads) {
    const size_t n = (size_t)units * kv_heads * kTicketStride * sizeof(int32_t);
    return (n + 255) / 256 * 256;
}

bool attn_vec_supported(pkv_dtype dtype, int32_t head_dim, int32_t group) {
    return (dtype == PKV_F32 || dtype == PKV_BF16) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && group >= 1 && group <= 8;
}

template <typename T, int D, int GT>
static hipError_t launch_vec_t(const AttnParams& p, hipStream_t stream) {
    dim3 grid(p.kv_heads, p.vec_wgs, 1);
    if (p.mode == kColumn) {
        attn_vec_kernel<T, D, GT, false><<<grid, dim3(kThreads), 0, stream>>>(p);
    } else {
        attn_vec_kernel<T, D, GT, true><<<grid, dim3(kThreads), 0, stream>>>(p);
    }
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

hipError_t launch_zero_uncovered(const AttnParams& p, pkv_dtype dtype, int32_t head_dim,
                                 hipStream_t stream) {
    const int32_t row_bytes = p.q_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4);
    if (p.total_q <= 0) return hipSuccess;
    zero_uncovered_kernel<<<dim3((p.total_q + kZeroRows - 1) / kZeroRows), dim3(256), 0, stream>>>(p, row_bytes);
    return hipGetLastError();
}

}  // namespace pkv
