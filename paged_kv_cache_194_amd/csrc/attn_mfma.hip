// Matrix-core (MFMA) attention for units with several query rows: chunked
// prefill segments and draft-verify blocks, and the single-row units of bf16
// calls whose GQA group is 8 or more.
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
// for a kv head is used by all of its query heads.  A work group (NW waves of
// RT row tiles of 16) takes BM = 16*NW*RT of those rows and a range of
// BN-key chunks (the launch shapes below).
//
// Per chunk the work group stages K and V row-major in LDS -- keys outside
// the rows' union of visible ranges, or without storage, are staged as zeros --
// and each wave runs two bf16 MFMA passes for each of its 16-row tiles with
// v_mfma_f32_16x16x32_bf16:
//   S^T[key][row] = K . Q^T     (A = K from LDS, B = Q^T from registers)
//   O^T[d][row]  += V^T . P^T   (A = V^T built by transposing LDS reads,
//                                ds_read_b64_tr_b16; B = P^T straight from the
//                                C layout of S^T)
// Chunks go from global memory straight into a ring of NS LDS stages
// (direct-to-LDS loads), NS - 1 chunks ahead of the one being computed.
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

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 8-byte chunks named by lanes 4m + i / 4, m = 0..3 (a 4 x 4 transpose
// of 16-bit elements per group).
__device__ __forceinline__ v4i16 ds_read_tr16(const uint8_t* lds) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(lds));
}
__device__ __forceinline__ uint32_t pair_bits(const v4i16& v, int h) {
    return (uint32_t)(uint16_t)v[2 * h] | ((uint32_t)(uint16_t)v[2 * h + 1] << 16);
}

constexpr int kIdWindow = 1024;   // block ids staged in LDS at a time
// Slack of the softmax reference point, in log2 units (probabilities < 256).
constexpr float kLazyLog2 = 8.f;


// Direct-to-LDS 16-byte load (global_load_lds_dwordx4): lane i's 16 bytes from
// `src` land at LDS byte address lds + 16*i (lds wave-uniform, through M0).
// Issued from inline assembly so that the compiler's wait-count bookkeeping
// does not serialize it; the kernel places its own waits.  STREAM: nontemporal
// (streaming) cache policy, for keys no other work group of the call reads.
// The same load from the wave-uniform base `sbase` (an SGPR pair) plus this
// lane's 32-bit byte offset `voff`.
template <bool STREAM>
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
    if constexpr (STREAM) {
        asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
    } else {
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
    }
}
// A 64-bit value known to be wave-uniform, moved to scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}
template <bool STREAM>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
    if constexpr (STREAM) {
        asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds) : "memory");
    } else {
        asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
    }
}
// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Source of the bytes staged for a key that is not wanted or has no storage.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[512];

// Launch shape per head_dim: NW waves, each owning RT tiles of 16 query rows
// (every K/V fragment a wave reads from LDS feeds RT MFMAs), chunks of BN
// keys, NS LDS stages (NS - 1 chunks in flight while one is computed), at
// least WPE waves per SIMD (a register cap).  Measured on the chunked-prefill
// and draft-verify workloads: with two row tiles a D = 128 wave fits two to a
// SIMD and two 68 KiB work groups share a CU; at D = 256 two row tiles do not
// fit two waves to a SIMD, and eight one-tile waves win, with two stages of
// 64-key chunks (draft verify 428 -> 407 us against four stages of 32 keys,
// once the per-chunk instruction count had been cut).
// FEW: calls whose units have at most 64 rows (max_seqlen_q * group: decode
// with a GQA group of 8 or 16) at D = 128 and 256.  There every row sits in
// the first wave and the chunk stream binds, so four one-tile waves with two
// stages make a 68 KiB work group and two share a CU: at D = 256 a call of 16
// splits of 4 sequences and 8 kv heads then fits one dispatch round (4 x
// 32K/64K keys, G 8: 339 -> 276 us); at D = 128 the first wave computes one
// row tile instead of two, empty, ones (same call: 178 -> 155 us).
template <int D, bool FEW = false>
struct MfmaShape;
template <>
struct MfmaShape<64> { static constexpr int NW = 4, RT = 2, BN = 64, NS = 4, WPE = 2; };
template <>
struct MfmaShape<128> { static constexpr int NW = 4, RT = 2, BN = 64, NS = 2, WPE = 2; };
template <>
struct MfmaShape<128, true> { static constexpr int NW = 4, RT = 1, BN = 64, NS = 2, WPE = 2; };
template <>
struct MfmaShape<256> { static constexpr int NW = 8, RT = 1, BN = 64, NS = 2, WPE = 1; };
template <>
struct MfmaShape<256, true> { static constexpr int NW = 4, RT = 1, BN = 32, NS = 2, WPE = 2; };
static_assert(16 * MfmaShape<128, true>::NW * MfmaShape<128, true>::RT ==
                  16 * MfmaShape<256, true>::NW * MfmaShape<256, true>::RT,
              "one row bound for the few-rows shapes");

template <int D, int NW, int RT, int BN, int NS>
struct MfmaCfg {
    static constexpr int NT = 64 * NW;            // threads
    static constexpr int BM = 16 * NW * RT;       // query rows per work group
    static constexpr int RB = D * 2;              // bytes per key row (one head)
    static constexpr int RC = D / 8;              // 16-byte columns per row
    static constexpr int CB = BN * RB;            // bytes of one chunk of K (or V)
    static constexpr int NI = CB / 1024;          // 1 KiB wave loads per chunk of K (or V)
    static constexpr int IPW = NI / NW;           // ... per wave
    static constexpr int KT = BN / 16;            // 16-key tiles per chunk
    static constexpr int KS = D / 32;             // k-steps of the QK product
    static constexpr int DT = D / 16;             // 16-wide d tiles of O
    static_assert(NI % NW == 0 && IPW >= 1, "chunk must split evenly over waves");
    static_assert(BN % 32 == 0, "PV k-steps take 32 keys");
    static_assert(RB <= 512, "zero row covers one key row");
    // Rows are stored unpadded with their 16-byte columns permuted by the row:
    // XOR with 2*row inside each group of 16 columns (D >= 128), rotation by
    // the row within the 8 columns (D = 64).  Measured on gfx950 with the
    // kernel's two read patterns (16-row ds_read_b128 for K, ds_read_b64_tr_b16
    // for V), either leaves no LDS bank conflicts.  swz maps a logical column
    // to its stored place; unswz is the inverse.
    __device__ static int swz(int r, int c) {
        if constexpr (RC >= 16) return c ^ ((2 * r) & 15);
        else return (c + r) & (RC - 1);
    }
    __device__ static int unswz(int r, int c) {
        if constexpr (RC >= 16) return c ^ ((2 * r) & 15);
        else return (c - r) & (RC - 1);
    }
};

// Keys one row tile of a unit needs: the union of its rows' visible ranges,
// from a 16-aligned start, in chunks of `bn` keys.  Row i of a unit of L rows
// over E keys sits at position E - L + i (causal: keys up to it; window W:
// the W keys ending there; left-padding bound `pad` > 0: no key before it,
// and a row before it keeps only its own key).  Both bounds are
// non-decreasing in i, so a tile's union runs from its first row's lower
// bound to its last row's upper bound.
struct TileKeys {
    int32_t key_lo, key_hi, c_base, nchunk;
};
__device__ __forceinline__ int32_t row_lo(const AttnParams& p, int32_t E, int32_t L, int32_t i,
                                          int32_t pad) {
    const int32_t pos = E - L + i;
    if (pad > 0 && pos < pad) return pos > 0 ? pos : 0;
    int32_t lo = 0;
    if (p.window > 0) {
        lo = pos - p.window + 1;
        lo = lo > 0 ? lo : 0;
    }
    return lo > pad ? lo : (pad > 0 ? pad : lo);
}
__device__ __forceinline__ int32_t row_hi(const AttnParams& p, int32_t E, int32_t L, int32_t i,
                                          int32_t pad) {
    const int32_t pos1 = E - L + i + 1;
    if ((pad > 0 && pos1 <= pad) || p.causal) return pos1 < E ? (pos1 > 0 ? pos1 : 0) : E;
    return E;
}
__device__ __forceinline__ TileKeys tile_keys(const AttnParams& p, int32_t E, int32_t L, int32_t M,
                                              int32_t m0, int32_t bm, int32_t bn, int32_t pad) {
    const int32_t G = p.group;
    const int32_t m_last = min(M, m0 + bm) - 1;
    TileKeys t;
    t.key_lo = row_lo(p, E, L, m0 / G, pad);
    t.key_hi = max(row_hi(p, E, L, m_last / G, pad), t.key_lo);
    t.c_base = (t.key_lo >> 4) << 4;
    t.nchunk = t.key_hi > t.c_base ? (t.key_hi - t.c_base + bn - 1) / bn : 0;
    return t;
}
// Chunks of row tile `tile` of unit u on the matrix-core path, or -1 when that
// (unit, tile) is not this path's work.
__device__ __forceinline__ int32_t mfma_item_chunks(const AttnParams& p, int32_t u, int32_t tile,
                                                    int32_t bm, int32_t bn) {
    const UnitInfo ui = load_unit(p, u);
    const int32_t L = ui.q_len;
    if (L <= 0 || (L == 1 && p.group <= 8 && !p.mfma_single)) return -1;
    const int32_t M = (L < p.max_seqlen_q ? L : p.max_seqlen_q) * p.group;
    if (tile * bm >= M) return -1;
    return tile_keys(p, ui.keys_ok ? ui.kv_end : 0, L, M, tile * bm, bm, bn, ui.pad).nchunk;
}

template <int D, int NW, int RT, int BN, int NS, int WPE, bool PAGED, bool STREAM>
__global__ __launch_bounds__(64 * NW, WPE) void attn_mfma_kernel(AttnParams p) {
    using C = MfmaCfg<D, NW, RT, BN, NS>;
    constexpr bool kMfmaPrio = D <= 128;
    constexpr int NT = C::NT, BM = C::BM, RB = C::RB, RC = C::RC, CB = C::CB, IPW = C::IPW,
                  KT = C::KT, KS = C::KS, DT = C::DT;

    // Stage s holds one chunk: K rows at sKV[s][0], V rows at sKV[s][CB].
    __shared__ __attribute__((aligned(1024))) uint8_t sKV[NS][2 * CB];
    __shared__ int32_t sIds[kIdWindow];
    __shared__ int32_t sLast;

    __shared__ int32_t sWork[5];
    const int32_t T = p.mfma_tiles;               // row tiles per (unit, kv head)
    // kv head fastest: the work groups reading the heads of the same keys run
    // together.  Those of kv head 0 also zero their share of uncovered rows.
    const int32_t g = blockIdx.x;
    if (p.zero_rows && g == 0) zero_rows_share(p, p.q_heads * D * 2, reinterpret_cast<uint32_t*>(&sLast), NT);
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int lr = lane & 15;                     // this lane's query row within the wave
    const int lq = lane >> 4;                     // lane group 0..3

    // Work items are (unit, row tile).  With one split, slot blockIdx.y of
    // unit blockIdx.z is row tile blockIdx.y.  With several, the
    // mfma_splits * items slots of a kv head are dealt over the items (a call
    // of one item included): an item of n chunks gets max(1, ceil(n / c))
    // consecutive slots, c the smallest chunk count per slot for which the
    // deal fits the grid.
    int32_t u, tile, split, S, slot0;
    if (p.mfma_splits == 1) {
        S = 1;
        tile = blockIdx.y;
        split = 0;
        u = blockIdx.z;
        slot0 = u * T + tile;
    } else {
        if (wave == 0) {
            const int32_t NI = p.num_units * T;
            const int32_t per = (NI + 63) / 64;
            const int32_t ib = lane * per, ie = min(NI, ib + per);
            auto item_n = [&](int32_t it) { return mfma_item_chunks(p, it / T, it - (it / T) * T, BM, BN); };
            const DealItems items = deal_items(item_n, ib, ie);
            const int32_t c = deal_size(items, item_n, (int64_t)p.mfma_splits * NI);
            int32_t cnt = 0;
            deal_for_each(items, item_n, [&](int32_t, int32_t n) { cnt += deal_slots_of(n, c); });
            int32_t incl = cnt;
#pragma unroll
            for (int st = 1; st < 64; st *= 2) {
                const int32_t y = __shfl_up(incl, st, 64);
                if (lane >= st) incl += y;
            }
            if (lane == 0) sWork[0] = -1;
            int32_t acc = incl - cnt;
            const int32_t w = blockIdx.y;
            deal_for_each(items, item_n, [&](int32_t it, int32_t n) {
                const int32_t k = deal_slots_of(n, c);
                if (w >= acc && w < acc + k) {
                    sWork[0] = it / T; sWork[1] = it - (it / T) * T; sWork[2] = w - acc; sWork[3] = k; sWork[4] = acc;
                }
                acc += k;
            });
        }
        __syncthreads();
        u = sWork[0]; tile = sWork[1]; split = sWork[2]; S = sWork[3]; slot0 = sWork[4];
        if (u < 0) return;                          // a spare slot
    }

    const UnitInfo ui = load_unit(p, u);
    const int32_t G = p.group;
    const int32_t L = ui.q_len;
    // Units with one row and a small group belong to the vector path, unless
    // this call runs everything here (mfma_single).
    if (L <= 0 || (L == 1 && G <= 8 && !p.mfma_single)) return;
    const int32_t Lr = L < p.max_seqlen_q ? L : p.max_seqlen_q;   // rows past the bound: uncovered
    const int32_t M = Lr * G;
    const int32_t m0 = tile * BM;
    if (m0 >= M) return;
    const int32_t E = ui.keys_ok ? ui.kv_end : 0;
    const int32_t Hkv = p.kv_heads;
    // A unit whose rows fit one tile has its keys read by one work group per
    // kv head: they stream past the caches even when other units' tiles share
    // theirs (column-store step 315-318 -> 311-313 us).
    const bool own_keys = M <= BM;

    // The union of this tile's rows' visible ranges, cut into S parts.
    const int32_t pad = ui.pad;
    const TileKeys tk = tile_keys(p, E, L, M, m0, BM, BN, pad);
    const int32_t key_lo = tk.key_lo, key_hi = tk.key_hi, c_base = tk.c_base, nchunk = tk.nchunk;
    auto lo_of = [&](int32_t i) __attribute__((always_inline)) -> int32_t { return row_lo(p, E, L, i, pad); };
    auto hi_of = [&](int32_t i) __attribute__((always_inline)) -> int32_t { return row_hi(p, E, L, i, pad); };
    const int32_t cps = (nchunk + S - 1) / S;
    const int32_t c_first = split * cps;
    const int32_t c_end = min(nchunk, c_first + cps);

    // This lane's rows: row lr of the wave's tiles rt = 0 .. RT-1.
    int32_t my_i[RT], my_h[RT], my_lo[RT], my_hi[RT];
    bool in_rows[RT], rows_ok[RT];
    u32x4 qf[RT][KS];                             // Q^T operand: d = ks*32 + 8*lq .. +7
    // Scores are scaled inside the exponent's fma by |scale|; a negative scale
    // flips the sign of q instead (exact in bf16).
    const float sc = fabsf(p.scale_log2);
    const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int32_t mm = m0 + (wave * RT + rt) * 16 + lr;
        const bool row_ok = mm < M;
        rows_ok[rt] = row_ok;
        my_i[rt] = row_ok ? mm / G : 0;
        my_h[rt] = row_ok ? mm - my_i[rt] * G : 0;
        my_lo[rt] = lo_of(my_i[rt]);
        my_hi[rt] = row_ok ? hi_of(my_i[rt]) : 0;
        in_rows[rt] = row_ok && (ui.q_start + my_i[rt]) >= 0 && (ui.q_start + my_i[rt]) < p.total_q;
        const uint8_t* qb = (const uint8_t*)p.q +
                            (((int64_t)(ui.q_start + my_i[rt]) * p.q_heads + (int64_t)g * G + my_h[rt]) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (in_rows[rt]) {
                const u32x4 x = ld16(qb + (ks * 32 + 8 * lq) * 2);
                qf[rt][ks] = u32x4{x.x ^ qsign, x.y ^ qsign, x.z ^ qsign, x.w ^ qsign};
            } else {
                qf[rt][ks] = u32x4{0u, 0u, 0u, 0u};
            }
    }
    // Q complete before the pipeline starts: otherwise the first use of qf in the
    // chunk loop would wait for every load in flight.
    wait_vm_all();
    // A wave none of whose rows exist (a unit of few rows, e.g. one query row
    // of a small group) still issues its share of every chunk's loads and
    // meets every barrier, but skips the products.
    bool any_row = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) any_row |= rows_ok[rt];
    const bool wave_idle = __ballot(any_row) == 0;

    f32x4_t o[RT][DT];
    float m_run[RT], l_run[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
    }

    const uint8_t* __restrict__ Kg = (const uint8_t*)p.k;
    const uint8_t* __restrict__ Vg = (const uint8_t*)p.v;
    const int64_t tok_stride = (int64_t)Hkv * D * 2;
    const int64_t head_off = (int64_t)g * D * 2;
    int32_t id_base = -kIdWindow;                 // first block of the staged id window

    // Issue chunk c (of this work group's range; past c_end nothing is wanted)
    // into stage st: wave loads w, w + NW, ... of K and of V.  Lane i of wave
    // load I fills stored place I*64 + i of the chunk: row r, stored column cs,
    // which holds logical column unswz(r, cs) of key c0 + r.  All addresses are
    // formed first (the block-id reads from LDS then overlap), and only then
    // are the loads issued.  c0 is a multiple of 16, so key c0 + r lies in
    // block (c0 >> 4) + (r >> 4) at slot r & 15; a ring row is found from one
    // modulo per chunk.  A key not wanted, or without storage, reads the zero row.
    const int64_t blk_stride = 16 * tok_stride;
    // Blocks without storage: bit KT*st + k is set when 16-key tile k of the
    // chunk in stage st has a block-table entry outside the pool.  Those keys
    // are staged from the zero row and must also be kept out of every row's
    // softmax, like keys outside its range.  Wave-uniform; each stage's bits
    // are set when its chunk is issued and read when it is computed.
    static_assert(KT * NS <= 32, "storage mask bits");
    uint32_t nostore = 0u;
    // Load m of this lane in a chunk that takes the uniform-base path: the
    // byte offset from the chunk's base, fixed for the whole loop.  Every
    // wave load covers rows of one 16-key tile (64 / RC rows, RC a power of
    // two dividing 64).
    static_assert(64 % RC == 0 && 16 % (64 / RC) == 0, "a wave load stays inside one 16-key tile");
    const int64_t row_stride = (int64_t)p.cols * tok_stride;        // ring: bytes per store row
    uint32_t issue_off[IPW];
#pragma unroll
    for (int m = 0; m < IPW; ++m) {
        const int place = (wave + NW * m) * 64 + lane;
        const int r = place / RC, cs = place - (place / RC) * RC;
        const int64_t o = PAGED ? (int64_t)(r & 15) * tok_stride + head_off + C::unswz(r, cs) * 16
                                : (int64_t)r * row_stride + head_off + C::unswz(r, cs) * 16;
        issue_off[m] = (uint32_t)o;
    }
    // The lane offsets must fit the 32-bit offset of the uniform-base path.
    const bool offs_fit = (PAGED ? (int64_t)15 * tok_stride : (int64_t)(BN - 1) * row_stride) + head_off + RB <
                          ((int64_t)1 << 31);
    auto issue = [&](int32_t c, int st) __attribute__((always_inline)) {
        const int32_t c0 = c_base + c * BN;
        const bool chunk_ok = c < c_end;
        // A chunk inside every row's range whose keys all have storage (and,
        // in a ring, do not wrap) is issued from one wave-uniform base per
        // load plus the lane's fixed offset, with no per-lane address work.
        bool fast = chunk_ok && c0 >= key_lo && c0 + BN <= key_hi;
        int32_t tid_k[KT];
        if constexpr (PAGED) {
            uint32_t bad = 0u;
            if (chunk_ok) {
#pragma unroll
                for (int k = 0; k < KT; ++k) {
                    int32_t w = (c0 >> 4) + k - id_base;
                    w = w < 0 ? 0 : (w >= kIdWindow ? kIdWindow - 1 : w);
                    const int32_t id = sIds[w];
                    tid_k[k] = id;
                    bad |= (id >= 0 && id < p.num_blocks) ? 0u : (1u << k);
                }
            }
            const uint32_t field = ((1u << KT) - 1u) << (KT * st);
            nostore = (nostore & ~field) | (bad << (KT * st));
            fast = fast && bad == 0u && offs_fit;
        }
        const uint32_t kdst = lds_addr(&sKV[st][0]), vdst = lds_addr(&sKV[st][CB]);
        int32_t ring0 = 0;
        if constexpr (!PAGED) {
            ring0 = c0 % p.rows;
            fast = fast && offs_fit && ring0 + BN <= p.rows;
        }
        if (fast) {
#pragma unroll
            for (int m = 0; m < IPW; ++m) {
                const int I = wave + NW * m;
                int64_t a;
                if constexpr (PAGED) {
                    const int tile = (I * (64 / RC)) >> 4;          // the 16-key tile of load m
                    a = (int64_t)__builtin_amdgcn_readfirstlane(tid_k[tile]) * blk_stride;
                } else {
                    a = (int64_t)ring0 * row_stride + (int64_t)ui.col * tok_stride;
                }
                const uint8_t* kb = uniform_ptr(Kg + a);
                const uint8_t* vb = uniform_ptr(Vg + a);
                const uint32_t km = (uint32_t)__builtin_amdgcn_readfirstlane((int)(kdst + I * 1024));
                const uint32_t vm = (uint32_t)__builtin_amdgcn_readfirstlane((int)(vdst + I * 1024));
                if (STREAM || own_keys) {
                    dma16s<true>(issue_off[m], kb, km);
                    dma16s<true>(issue_off[m], vb, vm);
                } else {
                    dma16s<false>(issue_off[m], kb, km);
                    dma16s<false>(issue_off[m], vb, vm);
                }
            }
            return;
        }
        const uint8_t* ks[IPW];
        const uint8_t* vs[IPW];
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            const int I = wave + NW * m;
            const int place = I * 64 + lane;
            const int r = place / RC, cs = place - (place / RC) * RC;
            const int32_t j = c0 + r;
            const bool want = chunk_ok && j >= key_lo && j < key_hi;
            int64_t a;
            if constexpr (PAGED) {
                int32_t w = (c0 >> 4) + (r >> 4) - id_base;
                w = w < 0 ? 0 : (w >= kIdWindow ? kIdWindow - 1 : w);
                const int32_t id = sIds[w];
                const bool ok = want && id >= 0 && id < p.num_blocks;
                a = ok ? (int64_t)id * blk_stride + (r & 15) * tok_stride + head_off : -1;
            } else {
                int32_t row = ring0 + r;
                if (row >= p.rows) row -= p.rows;
                if (row >= p.rows) row %= p.rows;         // rings shorter than a chunk
                a = want ? ((int64_t)row * p.cols + ui.col) * tok_stride + head_off : -1;
            }
            const int off = C::unswz(r, cs) * 16;
            ks[m] = a >= 0 ? Kg + a + off : kZeroRow + off;
            vs[m] = a >= 0 ? Vg + a + off : kZeroRow + off;
        }
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            const int I = wave + NW * m;
            const uint32_t km = (uint32_t)__builtin_amdgcn_readfirstlane((int)(kdst + I * 1024));
            const uint32_t vm = (uint32_t)__builtin_amdgcn_readfirstlane((int)(vdst + I * 1024));
            if (STREAM || own_keys) {
                dma16<true>(ks[m], km);
                dma16<true>(vs[m], vm);
            } else {
                dma16<false>(ks[m], km);
                dma16<false>(vs[m], vm);
            }
        }
    };
    // Stage the block ids of [blk, blk + kIdWindow) (paged): every thread calls it.
    auto stage_ids = [&](int32_t blk) __attribute__((always_inline)) {
        __syncthreads();
        for (int k = tid; k < kIdWindow; k += NT) {
            const int32_t b = blk + k;
            sIds[k] = (b < p.max_blocks && b >= 0) ? p.block_table[(int64_t)u * p.max_blocks + b] : -1;
        }
        id_base = blk;
        __syncthreads();
    };
    auto ensure_ids = [&](int32_t c) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const int32_t b_lo = (c_base + c * BN) >> 4;
            const int32_t b_hi = (c_base + c * BN + BN - 1) >> 4;
            if (b_lo < id_base || b_hi >= id_base + kIdWindow) stage_ids(b_lo);
        }
    };

    // LDS byte offsets of this lane's reads inside a stage, for key tile 0 and
    // PV step 0: the swizzle of a row depends on the row modulo 16 (column XOR)
    // or 8 (rotation) only, so later key tiles and PV steps add whole 16-row
    // blocks, an immediate offset of the read.
    int32_t k_off[KS], v_off[DT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_off[ks] = lr * RB + C::swz(lr, ks * 4 + lq) * 16;
    {
        const int vr0b = 4 * lq + (lr >> 2);
        const int half = (lr & 1) * 8;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) v_off[dt] = vr0b * RB + C::swz(vr0b, 2 * dt + ((lr & 3) >> 1)) * 16 + half;
    }
    // (Recomputed at every read, these offsets cost the head_dim-256 draft pass
    // 2 %, and 12-22 more VGPRs.)

    // A wave issues its two MFMA passes at raised priority and its softmax at
    // the normal one, so that on a SIMD shared with a wave of another phase
    // the matrix core is fed first and the VALU work fills the gaps (the
    // per-chunk barrier otherwise keeps a work group's waves in step).
    // Column-store step with head_dim 128: 437 -> 411 us; not taken at
    // head_dim 256, where it measured no gain.
    // ---- S^T = K . Q^T for this wave's RT x 16 rows and one chunk's BN keys ----
    auto qk = [&](const uint8_t* sKb, f32x4_t (&st)[RT][KT]) __attribute__((always_inline)) {
        if constexpr (kMfmaPrio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) st[rt][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(sKb + kt * 16 * RB + k_off[ks]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) st[rt][kt] = mfma16(a, qf[rt][ks], st[rt][kt]);
            }
        }
        if constexpr (kMfmaPrio) __builtin_amdgcn_s_setprio(0);
    };
    // ---- online softmax of chunk c's scores st, then O^T += V^T . P^T ----
    auto softmax_pv = [&](int32_t c, int st_idx, const f32x4_t (&st)[RT][KT], const uint8_t* sVb)
        __attribute__((always_inline)) {
        const int32_t c0 = c_base + c * BN;
        const uint32_t bad = (nostore >> (KT * st_idx)) & ((1u << KT) - 1u);   // tiles without storage
        // ---- online softmax (row lr of tile rt; keys kt*16 + 4*lq + e) ----
        // A chunk inside every row's visible range (the common case) needs no
        // per-key mask: a wave-uniform test picks that path.  Rows past M are
        // never written, so they do not force the mask.
        bool edge = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            edge |= rows_ok[rt] && !(my_lo[rt] <= c0 && c0 + BN <= my_hi[rt]);
        const bool masked = __ballot(edge) != 0 || bad != 0u;
        uint32_t pk[RT][KT][2];                   // probabilities, bf16, 4 keys per tile
        float alpha[RT];
        bool moved = false;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            uint32_t vis = ~0u;                   // bit kt*4 + e: key visible to this row
            float cmax = -INFINITY;
            if (masked) {
                vis = 0u;
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int32_t j = c0 + kt * 16 + 4 * lq + e;
                        const bool v = j >= my_lo[rt] && j < my_hi[rt] && !((bad >> kt) & 1u);
                        vis |= (v ? 1u : 0u) << (kt * 4 + e);
                        cmax = v ? fmaxf(cmax, st[rt][kt][e]) : cmax;
                    }
            } else {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) cmax = fmaxf(cmax, st[rt][kt][e]);
            }
            cmax = swap_op16<true>(cmax);
            cmax = swap_op32<true>(cmax);
            const float cm = cmax == -INFINITY ? -INFINITY : cmax * sc;   // scaled, log2 units
            // The row's reference point moves only when a chunk's maximum
            // passes it by more than kLazyLog2: probabilities stay below
            // 2^kLazyLog2 (exact in the fp32 sums, the same relative rounding
            // in bf16), and most chunks skip the rescale of O.
            const bool bump = cm > m_run[rt] + kLazyLog2;
            const float m_new = bump ? cm : m_run[rt];
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            alpha[rt] = bump ? fast_exp2(m_run[rt] - m_use) : 1.f;
            moved |= bump;
            m_run[rt] = m_new;
            float psum = 0.f;
            // keep(kt, e): key kt*4 + e of the lane enters the sums.  Unmasked
            // chunks (wave-uniform) take an instantiation with no per-key test.
            auto probs = [&](auto keep) __attribute__((always_inline)) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    float pr[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = fmaf(st[rt][kt][e], sc, -m_use);
                        pr[e] = fast_exp2(keep(kt, e) ? x : -INFINITY);
                    }
                    // rounded to bf16 for the MFMA; the row sum adds the same rounded values
                    pk[rt][kt][0] = pack_bf16(pr[0], pr[1]);
                    pk[rt][kt][1] = pack_bf16(pr[2], pr[3]);
                    psum = dot2_bf16(pk[rt][kt][0], kBf16OnePair, psum);
                    psum = dot2_bf16(pk[rt][kt][1], kBf16OnePair, psum);
                }
            };
            if (masked) probs([&](int kt, int e) { return ((vis >> (kt * 4 + e)) & 1u) != 0u; });
            else probs([](int, int) { return true; });
            l_run[rt] = l_run[rt] * alpha[rt] + psum;
        }
        if (__ballot(moved) != 0) {               // some row's max moved
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    o[rt][dt][0] *= alpha[rt]; o[rt][dt][1] *= alpha[rt];
                    o[rt][dt][2] *= alpha[rt]; o[rt][dt][3] *= alpha[rt];
                }
        }
        if constexpr (kMfmaPrio) __builtin_amdgcn_s_setprio(1);
        // ---- O^T += V^T . P^T, 32 keys per step: tiles (2s, 2s+1) ----
#pragma unroll
        for (int s2 = 0; s2 < KT / 2; ++s2) {
            u32x4 b[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                b[rt] = u32x4{pk[rt][2 * s2][0], pk[rt][2 * s2][1], pk[rt][2 * s2 + 1][0], pk[rt][2 * s2 + 1][1]};
            // A = V^T rows d = dt*16 + lr, keys {kk0..kk0+3, kk0+16..kk0+19},
            // kk0 = s2*32 + 4*lq: two transposing reads of row-major V; lane
            // (4m + c) of a 16-lane group names row kk0 + m, elements
            // dt*16 + 4c .. +3 (8 bytes of a 16-byte column).
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const v4i16 lo4 = ds_read_tr16(sVb + s2 * 32 * RB + v_off[dt]);
                const v4i16 hi4 = ds_read_tr16(sVb + (s2 * 32 + 16) * RB + v_off[dt]);
                const u32x4 a = u32x4{pair_bits(lo4, 0), pair_bits(lo4, 1), pair_bits(hi4, 0), pair_bits(hi4, 1)};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) o[rt][dt] = mfma16(a, b[rt], o[rt][dt]);
            }
        }
    };

    // Chunk i of this work group (i = 0 .. n-1) is chunk c_first + i, staged
    // in stage i % NS.  Step i: wait for this wave's loads of chunk i
    // (the loads of the NS - 2 later chunks stay in flight), barrier (all
    // waves' loads of chunk i have landed; every wave is done with chunk i-1),
    // issue chunk i + NS - 1 into chunk i-1's stage, compute chunk i.
    // Loads past the range read the zero row, so every step waits for the
    // same count.
    const int32_t n = c_end > c_first ? c_end - c_first : 0;
    if (n > 0) {
#pragma unroll
        for (int s = 0; s < NS - 1; ++s) {
            if (s < n) ensure_ids(c_first + s);
            issue(c_first + s, s);
        }
        for (int32_t i = 0; i < n; ++i) {
            wait_vm<2 * IPW * (NS - 2)>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (i + NS - 1 < n) ensure_ids(c_first + i + NS - 1);
            issue(c_first + i + NS - 1, (i + NS - 1) % NS);
            const int st = i % NS;
            if (!wave_idle) {
                f32x4_t sc4[RT][KT];
                qk(&sKV[st][0], sc4);
                softmax_pv(c_first + i, st, sc4, &sKV[st][CB]);
            }
        }
        wait_vm<0>();                             // no load may land after the work group ends
    }

    // Row sums across the 4 lane groups.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        l_run[rt] = swap_op16<false>(l_run[rt]);
        l_run[rt] = swap_op32<false>(l_run[rt]);
    }

    // This lane holds O^T[d][row] for d = dt*16 + 4*lq + e of each of its rows.
    if (S == 1) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (!in_rows[rt]) continue;
            const int64_t orow = ((int64_t)(ui.q_start + my_i[rt]) * p.q_heads + (int64_t)g * G + my_h[rt]) * D;
            const float inv = l_run[rt] > 0.f ? 1.f / l_run[rt] : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = dt * 16 + 4 * lq;
                const uint2 w2 = uint2{pack_bf16(o[rt][dt][0] * inv, o[rt][dt][1] * inv),
                                       pack_bf16(o[rt][dt][2] * inv, o[rt][dt][3] * inv)};
                *reinterpret_cast<uint2*>((uint16_t*)p.out + orow + d) = w2;
            }
        }
        return;
    }

    // ---- split-K partials: [slot][kv head][BM][D] and (m, l) ----
    const int64_t wi = (int64_t)(slot0 + split) * Hkv + g;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rloc = (wave * RT + rt) * 16 + lr;
        float* po = p.mws_o + (wi * BM + rloc) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            st_agent2(po + dt * 16 + 4 * lq, o[rt][dt][0], o[rt][dt][1]);
            st_agent2(po + dt * 16 + 4 * lq + 2, o[rt][dt][2], o[rt][dt][3]);
        }
        if (lq == 0) st_agent2(&p.mws_ml[(wi * BM + rloc) * 2], m_run[rt], l_run[rt]);
    }
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
    const int64_t w0 = (int64_t)slot0 * Hkv + g;
    constexpr int CH = 16;
    for (int idx = tid; idx < BM * (D / 4); idx += NT) {
        const int r = idx / (D / 4), d4 = (idx - r * (D / 4)) * 4;
        const int32_t mm = m0 + r;
        if (mm >= M) continue;
        const int32_t ii = mm / G, hh = mm - (mm / G) * G;
        if (ui.q_start + ii < 0 || ui.q_start + ii >= p.total_q) continue;
        const float* osrc = p.mws_o + (w0 * BM + r) * D + d4;
        const float* msrc = p.mws_ml + (w0 * BM + r) * 2;
        const int64_t ostride = (int64_t)Hkv * BM * D, mstride = (int64_t)Hkv * BM * 2;
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

template <int D, bool FEW = false>
constexpr int32_t shape_rows() { return 16 * MfmaShape<D, FEW>::NW * MfmaShape<D, FEW>::RT; }

// Whether a call whose units have up to `rows` rows (max_seqlen_q * group)
// takes the few-rows shape.
static bool few_rows(int32_t head_dim, int64_t rows) {
    return (head_dim == 128 || head_dim == 256) && rows <= shape_rows<256, true>();
}

int32_t mfma_rows_per_group(int32_t head_dim, int64_t rows) {
    if (few_rows(head_dim, rows)) return head_dim == 128 ? shape_rows<128, true>() : shape_rows<256, true>();
    return head_dim == 64 ? shape_rows<64>() : head_dim == 128 ? shape_rows<128>() : shape_rows<256>();
}
// Work groups of the matrix-core kernel one CU holds at once (LDS and
// register budgets of the shape: 68 KiB / 2 waves per SIMD at D <= 128 and
// for the few-rows shape, 132 KiB at D = 256).
int32_t mfma_groups_per_cu(int32_t head_dim, int64_t rows) {
    return head_dim == 256 && !few_rows(head_dim, rows) ? 1 : 2;
}

int32_t mfma_chunk_keys(int32_t head_dim, int64_t rows) {
    if (few_rows(head_dim, rows)) return head_dim == 128 ? MfmaShape<128, true>::BN : MfmaShape<256, true>::BN;
    return head_dim == 64 ? MfmaShape<64>::BN : head_dim == 128 ? MfmaShape<128>::BN : MfmaShape<256>::BN;
}

bool attn_mfma_supported(pkv_dtype dtype, int32_t head_dim) {
    return dtype == PKV_BF16 && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

template <int D, bool FEW, bool STREAM>
static void launch_mfma_policy(const AttnParams& p, dim3 grid, hipStream_t stream) {
    using Sh = MfmaShape<D, FEW>;
    if (p.mode == kColumn) {
        attn_mfma_kernel<D, Sh::NW, Sh::RT, Sh::BN, Sh::NS, Sh::WPE, false, STREAM><<<grid, dim3(64 * Sh::NW), 0, stream>>>(p);
    } else {
        attn_mfma_kernel<D, Sh::NW, Sh::RT, Sh::BN, Sh::NS, Sh::WPE, true, STREAM><<<grid, dim3(64 * Sh::NW), 0, stream>>>(p);
    }
}

template <int D>
static hipError_t launch_mfma_t(const AttnParams& p, hipStream_t stream) {
    const bool dealt = p.mfma_splits > 1;
    dim3 grid(p.kv_heads, p.mfma_tiles * p.mfma_splits * (dealt ? p.num_units : 1), dealt ? 1 : p.num_units);
    // With one row tile per (unit, kv head) every key is staged by one work
    // group only, so the chunks stream past the caches (long-context decode
    // with a group of 8: 364 -> 338 us; draft verify 470 -> 460 us).  With
    // several row tiles, the tiles of a unit read the same keys and the cached
    // policy keeps them (the column-store step ran 3 % slower streamed); the
    // kernel still streams the keys of units whose rows fit one tile.
    if constexpr (D == 128 || D == 256) {
        if (few_rows(D, (int64_t)p.max_seqlen_q * p.group)) {
            if (p.mfma_tiles != 1) return hipErrorInvalidValue;     // one tile holds every row
            launch_mfma_policy<D, true, true>(p, grid, stream);
            return hipGetLastError();
        }
    }
    if (p.mfma_tiles == 1) launch_mfma_policy<D, false, true>(p, grid, stream);
    else launch_mfma_policy<D, false, false>(p, grid, stream);
    return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams& p, pkv_dtype dtype, int32_t head_dim, hipStream_t stream) {
    if (!attn_mfma_supported(dtype, head_dim)) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_mfma_t<64>(p, stream);
    if (head_dim == 128) return launch_mfma_t<128>(p, stream);
    return launch_mfma_t<256>(p, stream);
}

}  // namespace pkv
