// Dense prefill FMHA, bf16 in/out, on gfx950 bf16 MFMA with fp32 accumulation.
//
// Method: the fused, tiled attention of the TensorRT-LLM FMHA page
// (zyxy.net/?p=24414, section 2: score, softmax and weighted sum fused in one
// kernel, tiles staged on chip, a bank-conflict-free on-chip layout, stable
// softmax) with the online softmax update of FlashAttention (FlashDecoding++
// summary, wenjunhu.com/d/2311396.html, section 1), so the T x T score matrix
// never leaves registers.  K/V tiles are double-buffered in LDS: the next
// tile is fetched while the current one is consumed (the ping-pong buffer of
// the same summary, section 4).
//
// gfx950 mapping
// --------------
// A workgroup is 8 wavefronts = 256 query rows of one (batch, head); each
// wavefront owns 32 rows.  Per key tile of BN = 32 keys a wavefront does
//
//   S^T = K Q^T     8 x v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q held in
//                   VGPRs for the whole kernel.  Computing S^T rather than S
//                   gives lane l the scores of query row l % 32 for 16 of the
//                   32 keys (the other 16 sit in lane l ^ 32): row max and
//                   row sum are lane-local plus one v_permlane32_swap.
//   softmax         exp2 of the scaled scores against the running max, P
//                   rounded to bf16 (already in B-operand order for PV).
//   O^T += V^T P^T  8 MFMAs, A = V^T from LDS.
//
// MFMA and VALU work of one wavefront do not overlap on gfx950; those of two
// wavefronts on one SIMD do.  So the eight wavefronts form two groups (one
// wavefront of each per SIMD) that run half a tile apart: while group 0
// issues the MFMAs of tile t (PV of t-1, then S of t), group 1 runs the
// softmax of tile t-1, and the other way round.  A workgroup barrier
// separates the phases.  Each wavefront stays under 256 VGPRs (two per SIMD).
//
// LDS: K row-major with a 16-byte row pad (conflict-free 16-row reads, affine
// addresses).  V is transposed while it is written (V^T: one row per head
// dimension) with the keys of each 16-key group ordered so that the 8 keys
// one MFMA lane needs are 16 contiguous bytes; the 80-byte V^T row stride
// makes the 16-row reads conflict-free.  Even dimensions 2i take rows i and
// odd ones 2i + 1 rows D/2 + i: a thread that loads the dimension pair
// (2i, 2i + 1) then writes rows 80 bytes apart across the wavefront (16 bank
// offsets, a 2-way conflict) instead of 160 (8 offsets, 4-way).  O^T
// inherits the row order; the epilogue interleaves the two halves.
//
// The running max is raised (and O, l rescaled) only when a row's max grows
// by more than 2^8; otherwise exponentials are taken against the stale max.
// Results are identical in exact arithmetic (numerator and denominator share
// the reference) and every exponential stays <= 2^8.  The row sum adds the
// bf16-rounded P that the MFMA multiplies with V.
//
// Causal masking (key j visible to query i iff j <= i + Tk - Tq) is applied
// only on tiles that cross the diagonal; tiles wholly above a wavefront's
// rows are skipped.  Workgroups are issued heaviest (longest key range)
// first, and all query tiles of one (b, h) land on one XCD so their shared
// K/V stay in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;         // 256 query rows per workgroup
constexpr int kBN = 32;                  // keys per tile
constexpr float kRescaleThresh = 8.0f;   // log2 units

template <int D>
struct Cfg {
    static constexpr int KS = D / 16;                    // MFMA k-steps of K Q^T
    static constexpr int DB = D / 32;                    // 32-row blocks of O^T (dims)
    static constexpr int CPR = D / 8;                    // 16-byte chunks per K row
    static constexpr int K_STRIDE = D * 2 + 16;          // K row + 16-byte pad
    static constexpr int K_BYTES = kBN * K_STRIDE;
    static constexpr int VT_STRIDE = kBN * 2 + 16;       // V^T row (32 keys) + pad
    static constexpr int V_BYTES = D * VT_STRIDE;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
    static constexpr int K_CHUNKS = kBN * CPR;           // 16-byte chunks per K tile
    static constexpr int V_UNITS = (kBN / 4) * (D / 2);  // 4-key x 2-dim V units
};

// V^T position of key k (0..31) in its row: in each 16-key group the 4-key
// blocks 1 and 2 trade places, so keys 16s + {0..3, 8..11} (MFMA lanes 0-31)
// and 16s + {4..7, 12..15} (lanes 32-63) are each contiguous.
__device__ __forceinline__ int vt_pos(int key) {
    const int a = (key >> 2) & 3;
    return (key & ~15) | ((((a & 1) << 1) | (a >> 1)) << 2) | (key & 3);
}

// One thread's share of a tile in flight: a 16-byte K chunk and a 4-key x
// 2-dim V unit (4 dwords).
struct Stage {
    u32x4 k;
    u32x4 v;
};

// Raw buffer resource over the rows [k0, min(k0 + kBN, Tk)) of one (b, h) K or
// V slice.  Buffer loads past its end return 0 without touching memory, so
// tail tiles, tiles past the key range and the idle threads of D = 64 need no
// branch and no address clamp; the descriptor is built with scalar ALU only.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data, no swizzle
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int k0, int Tk) {
    // (the clamp lowers to a vector op; readfirstlane keeps the descriptor scalar)
    const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(kBN, Tk - k0)) * D * 2);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)k0 * D), (short)0, bytes,
                                             kRsrcWord3);
}

// Byte offsets of this thread's K chunk and V unit inside a tile (fixed for
// the whole kernel).  Threads past the tile's chunk count land past the
// descriptor's end and read zeros.
template <int D>
struct LoadOffsets {
    int k, v;
    __device__ explicit LoadOffsets(int tid) {
        constexpr int CPR = Cfg<D>::CPR;
        k = (tid / CPR) * D * 2 + 16 * (tid % CPR);
        v = 4 * (tid / (D / 2)) * D * 2 + 4 * (tid % (D / 2));   // keys 4kb4.., dims 2dp, 2dp+1
    }
};

template <int D>
__device__ __forceinline__ void load_stage(Stage& st, const uint16_t* __restrict__ kp,
                                           const uint16_t* __restrict__ vp, int k0k, int k0v,
                                           int Tk, const LoadOffsets<D>& off) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc<D>(kp, k0k, Tk);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc<D>(vp, k0v, Tk);
    st.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off.k, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; j++) st.v[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, off.v + j * D * 2, 0, 0);
}

// Paged K/V (prefill against a paged cache, [pages][Hkv][16][D]): within a
// 32-key tile, the K rows of one wavefront's chunks (4 for D = 128, 8 for
// D = 64) and the keys of its V units (the same) lie in one 16-token page,
// slot 0 or 1 of the tile, so each wavefront loads through a descriptor
// over that page alone: its base from the sequence's block-table entry, its
// size the page's valid rows (a page at or past the sequence's length has
// none and reads zeros without touching memory).
struct PagedKV {
    const uint16_t* kpool;
    const uint16_t* vpool;
    const int32_t* table;   // this sequence's block-table row
    int Hkv, kvh, Tk;
    int slot_k, slot_v;     // this wavefront's page within a tile, -1 = no rows
};

template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* pool, const PagedKV& pk,
                                                            int k0, int slot) {
    const int p = k0 / 16 + max(slot, 0);
    const int valid = slot < 0 ? 0 : max(0, min(16, pk.Tk - p * 16));
    const int bytes = __builtin_amdgcn_readfirstlane(valid * D * 2);
    const uint16_t* base = pool;
    if (bytes > 0) {
        const int phys = __builtin_amdgcn_readfirstlane(pk.table[p]);
        base = pool + ((size_t)phys * pk.Hkv + pk.kvh) * 16 * D;
    }
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kRsrcWord3);
}

template <int D>
__device__ __forceinline__ void load_stage_paged(Stage& st, const PagedKV& pk, int k0k, int k0v,
                                                 const LoadOffsets<D>& off) {
    const __amdgpu_buffer_rsrc_t rk = page_rsrc<D>(pk.kpool, pk, k0k, pk.slot_k);
    const __amdgpu_buffer_rsrc_t rv = page_rsrc<D>(pk.vpool, pk, k0v, pk.slot_v);
    st.k = __builtin_amdgcn_raw_buffer_load_b128(rk, off.k, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; j++) st.v[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, off.v + j * D * 2, 0, 0);
}

template <int D>
__device__ __forceinline__ void store_stage(const Stage& st, unsigned char* kbuf,
                                            unsigned char* vbuf, int tid, bool do_k, bool do_v) {
    using C = Cfg<D>;
    if (do_k && tid < C::K_CHUNKS) {
        const int row = tid / C::CPR, ch = tid % C::CPR;
        *(u32x4*)(kbuf + row * C::K_STRIDE + 16 * ch) = st.k;
    }
    if (do_v && tid < C::V_UNITS) {
        const int dp = tid % (D / 2), kb4 = tid / (D / 2);
        // st.v[j] = (dim 2dp, dim 2dp+1) of key 4kb4 + j -> two V^T rows of 4 keys
        const uint32_t v0 = st.v[0], v1 = st.v[1], v2 = st.v[2], v3 = st.v[3];
        const uint32_t e01 = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        const uint32_t e23 = __builtin_amdgcn_perm(v3, v2, 0x05040100u);
        const uint32_t o01 = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
        const uint32_t o23 = __builtin_amdgcn_perm(v3, v2, 0x07060302u);
        unsigned char* row = vbuf + C::K_BYTES + dp * C::VT_STRIDE + vt_pos(4 * kb4) * 2;
        *(u32x2*)row = u32x2{e01, e23};                             // dim 2dp: row dp
        *(u32x2*)(row + (D / 2) * C::VT_STRIDE) = u32x2{o01, o23};  // dim 2dp + 1: row D/2 + dp
    }
}

template <int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                         float* __restrict__ lse, int BH, int Hq, int Hkv, int Tq, int Tk_dense,
                         int n_qtiles, float scale_log2, const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ kv_lens, int bt_stride) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::BUF_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
    const int li = lane & 31, hi = lane >> 5;
    // Wavefront w runs on SIMD w % 4; group 1 (waves 4-7) runs one phase
    // behind group 0.  Row blocks alternate between the groups so both see
    // the same share of the causal diagonal.
    const int grp = wave >> 2;
    const int rb = 2 * (wave & 3) + grp;

    // Heaviest query tiles first.  Workgroups are dealt to the 8 XCDs
    // round-robin, so id % 8 picks the XCD: with slot = id % BH, the kv group
    // kg = slot % (B * Hkv) and the head within the group g = slot / (B * Hkv),
    // every query tile of every head that reads one kv head's K/V lands on
    // one XCD (and its L2) when BH and B * Hkv are multiples of 8.  Without
    // grouped heads this is the identity, slot = b * Hq + h.
    const int id = blockIdx.x;
    const int slot = id % BH;
    const int qt = n_qtiles - 1 - id / BH;
    const int KG = (BH / Hq) * Hkv;      // (batch, kv head) groups
    const int kg = slot % KG, g_in = slot / KG;
    const int b = kg / Hkv, kvh = kg % Hkv, h = kvh * (Hq / Hkv) + g_in;
    const int bh = b * Hq + h;
    const int q0 = qt * kBM;
    const int qw0 = q0 + rb * 32;        // this wavefront's first row
    const int qrow = qw0 + li;           // the query row of this lane
    // paged: the sequence's own key count (its chunk of Tq queries is its
    // last Tq positions, so the causal diagonal sits at kv_len - Tq), clamped
    // to what its block-table row can map so no page index leaves the row
    const int Tk = PAGED ? __builtin_amdgcn_readfirstlane(max(0, min(kv_lens[b], bt_stride * 16)))
                         : Tk_dense;
    const int diag = Tk - Tq;

    const uint16_t* qp = q + (size_t)bh * Tq * D;
    const uint16_t* kp = PAGED ? k : k + (size_t)(b * Hkv + kvh) * Tk * D;
    const uint16_t* vp = PAGED ? v : v + (size_t)(b * Hkv + kvh) * Tk * D;

    // Q fragments (B operand of S^T = K Q^T): row qrow, dims 16s + 8hi .. +7.
    // Loaded unconditionally (clamped row, zeroed past Tq) so that no
    // exec-masked load is pending when the main loop starts.
    bf16x8 qf[C::KS];
    {
        const int qr = min(qrow, max(Tq - 1, 0));
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            u32x4 w = *(const u32x4*)(qp + (size_t)qr * D + 16 * s + 8 * hi);
            if (qrow >= Tq) w = u32x4{0, 0, 0, 0};
            qf[s] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // key range of the workgroup and of this wavefront
    int kend = Tk, kend_w = Tk;
    if (CAUSAL) {
        kend = max(0, min(Tk, q0 + kBM + diag));
        kend_w = max(0, min(Tk, qw0 + 32 + diag));
    }
    const int n_tiles = (kend + kBN - 1) / kBN;
    const int n_tiles_w = (kend_w + kBN - 1) / kBN;   // tiles with a visible key for this wavefront

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; db++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 sacc;
    bf16x8 pf[2];

    // Global phase p: group 0 runs its MFMA step t at p = 2t and its softmax
    // step t at p = 2t + 1; group 1 runs each one phase later.  K(t) lives in
    // buffer t % 2 during phases 2t and 2t+1 (the two groups' S(t)); V(t)
    // lives in buffer t % 2 during phases 2t+2 and 2t+3 (their PV(t)).  The
    // pair (K(t+1), V(t)) is loaded into register stage t % 2 at the start of
    // phase 2t - 2 and written to LDS at the end of phase 2t + 1, so every
    // load has four phases to arrive.
    // PV at t = 0 multiplies P = 0 with the V region of buffer 1: zero both so
    // that it adds exact zeros.
    pf[0] = pf[1] = bf16x8{};
    for (int i = tid; i < C::V_BYTES / 16; i += kThreads)
        *(u32x4*)(smem + C::BUF_BYTES + C::K_BYTES + 16 * i) = u32x4{0, 0, 0, 0};
    LoadOffsets<D> off(tid);
    PagedKV pk{};
    if constexpr (PAGED) {
        // first K row / V key of this wavefront's share of a tile
        const int rowk = (wave * 64) / C::CPR, rowv = 4 * ((wave * 64) / (D / 2));
        pk = PagedKV{kp, vp, block_table + (size_t)b * bt_stride, Hkv, kvh, Tk,
                     rowk < kBN ? rowk / 16 : -1, rowv < kBN ? rowv / 16 : -1};
        off.k -= max(pk.slot_k, 0) * 16 * D * 2;   // offsets within the page
        off.v -= max(pk.slot_v, 0) * 16 * D * 2;
    }
    Stage st0, st1;
    auto load_pair = [&](Stage& st, int t) {  // K(t+1), V(t)
        if constexpr (PAGED) load_stage_paged<D>(st, pk, (t + 1) * kBN, t * kBN, off);
        else load_stage<D>(st, kp, vp, (t + 1) * kBN, t * kBN, Tk, off);
    };
    auto store_pair = [&](const Stage& st, int t) {
        if (t < n_tiles)
            store_stage<D>(st, smem + ((t + 1) & 1) * C::BUF_BYTES, smem + (t & 1) * C::BUF_BYTES,
                           tid, t + 1 < n_tiles, true);
    };
    if (n_tiles > 0) {
        if constexpr (PAGED) load_stage_paged<D>(st0, pk, 0, 0, off);
        else load_stage<D>(st0, kp, vp, 0, 0, Tk, off);
        store_stage<D>(st0, smem, smem, tid, true, false);
    }
    __builtin_amdgcn_s_waitcnt(0);  // Q and the first K tile have landed
    load_pair(st0, 0);
    __syncthreads();

    // One step t of group G: its MFMA phase, then its softmax phase.  Every
    // global load is unconditional, so the wait before each LDS store covers
    // only the stage being stored, not the loads issued after it.
    // cur = stage t % 2 (pair t), nxt = stage (t + 1) % 2 (pair t + 1).
    auto step = [&](int t, Stage& cur, Stage& nxt, auto G) {
        constexpr int g = decltype(G)::value;
        // ---- MFMA step t (phase 2t for group 0, 2t+1 for group 1):
        //      O^T += V^T P^T for tile t-1 and S^T = K Q^T for tile t.
        if (g == 0) load_pair(nxt, t + 1);
        if (t <= n_tiles_w) {
            // All 16 LDS operands are requested first, V and K alternating in
            // the order the MFMAs consume them; PV(t-1) and S(t) MFMAs then
            // alternate too, so each waits only for its own operand and the S
            // chain's dependences are covered by PV MFMAs.  At t = 0 PV adds
            // P = 0 times the zeroed V buffer; at t = n_tiles_w S is computed
            // and not used.
            bf16x8 vf[C::KS], kf[C::KS];
            const unsigned char* sV = smem + ((t - 1) & 1) * C::BUF_BYTES + C::K_BYTES +
                                      li * C::VT_STRIDE + 16 * hi;
            const unsigned char* sK = smem + (t & 1) * C::BUF_BYTES + li * C::K_STRIDE + 16 * hi;
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                // V^T rows 32db + li; keys key(hi, 0..7) of step ps at positions 16ps + 8hi
                const int ps = s / C::DB, db = s % C::DB;
                vf[s] = *(const bf16x8*)(sV + 32 * db * C::VT_STRIDE + 32 * ps);
                kf[s] = *(const bf16x8*)(sK + 32 * s);
            }
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                const int ps = s / C::DB, db = s % C::DB;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], pf[ps], oacc[db], 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], s == 0 ? f32x16{} : sacc,
                                                               0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::KS, 0);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::KS, 0);  // then MFMAs
        }
        if (g == 1) store_pair(cur, t);
        __syncthreads();

        // ---- softmax step t (phase 2t+1 for group 0, 2t+2 for group 1)
        if (g == 1) load_pair(cur, t + 2);
        if (t < n_tiles_w) {
            const int k0 = t * kBN;
            // sacc[r] is the score of key k0 + 8(r/4) + 4hi + r%4
            if (k0 + kBN > Tk || (CAUSAL && k0 + kBN - 1 > qw0 + diag)) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int kj = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (kj >= Tk || (CAUSAL && kj > qrow + diag)) sacc[r] = -INFINITY;
                }
            }
            float mx;
            {   // max tree of depth 4 (v_max3)
                float t0 = __builtin_fmaxf(__builtin_fmaxf(sacc[0], sacc[1]), sacc[2]);
                float t1 = __builtin_fmaxf(__builtin_fmaxf(sacc[3], sacc[4]), sacc[5]);
                float t2 = __builtin_fmaxf(__builtin_fmaxf(sacc[6], sacc[7]), sacc[8]);
                float t3 = __builtin_fmaxf(__builtin_fmaxf(sacc[9], sacc[10]), sacc[11]);
                float t4 = __builtin_fmaxf(__builtin_fmaxf(sacc[12], sacc[13]), sacc[14]);
                t0 = __builtin_fmaxf(__builtin_fmaxf(t0, t1), t2);
                t3 = __builtin_fmaxf(__builtin_fmaxf(t3, t4), sacc[15]);
                mx = half_swap_max(__builtin_fmaxf(t0, t3));
            }
            mx = (mx == -INFINITY) ? -INFINITY : mx * scale_log2;
            const float m_new = fmaxf(m_run, mx);
            if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleThresh)) {
                const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; db++) oacc[db] *= alpha;
                m_run = m_new;
            }
            const float m_eff = (m_run == -INFINITY) ? 0.f : m_run;
            float l0 = l_run, l1 = 0.f;   // two row-sum chains
#pragma unroll
            for (int ps = 0; ps < 2; ps++) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float p0 = fast_exp2(__builtin_fmaf(sacc[8 * ps + 2 * e], scale_log2, -m_eff));
                    const float p1 = fast_exp2(__builtin_fmaf(sacc[8 * ps + 2 * e + 1], scale_log2, -m_eff));
                    w[e] = pack_bf16x2(p0, p1);
                    float& acc = (e & 1) ? l1 : l0;
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]),
                                                          __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
                }
                pf[ps] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
            l_run = l0 + l1;
        }
        if (g == 0) store_pair(cur, t);
        __syncthreads();
    };
    // The two groups run separate copies of the loop (the branch on grp is
    // wave-uniform); both pass the same number of barriers.
    // Steps run t = 0 .. n_tiles; the loop takes them in pairs (the stages
    // swap roles) and an odd last step runs after it, so that inside the
    // loop both steps are unconditional and the waits stay exact.
    if (grp == 0) {
        const std::integral_constant<int, 0> G0;
        int t = 0;
        for (; t + 1 <= n_tiles; t += 2) {
            step(t, st0, st1, G0);
            step(t + 1, st1, st0, G0);
        }
        if (t == n_tiles) step(t, st0, st1, G0);
        __syncthreads();  // group 1's last phase
    } else {
        const std::integral_constant<int, 1> G1;
        load_pair(st1, 1);  // phase 0: group 0 computes S(0); group 1 only loads
        __syncthreads();
        int t = 0;
        for (; t + 1 <= n_tiles; t += 2) {
            step(t, st0, st1, G1);
            step(t + 1, st1, st0, G1);
        }
        if (t == n_tiles) step(t, st0, st1, G1);
    }

    // ---- epilogue: O = O / l, lse = m ln2 + ln l ----------------------------
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < Tq) {
        // O^T row p = 32 db + 8 g + 4 hi + j holds dimension 2p (p < D/2) or
        // 2(p - D/2) + 1: rows p of block db and p + D/2 of block db + DB/2
        // give dimensions 2p and 2p + 1, so 4 rows make 16 contiguous bytes.
        uint16_t* op = o + ((size_t)bh * Tq + qrow) * D;
#pragma unroll
        for (int db = 0; db < C::DB / 2; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int p0 = 32 * db + 8 * g + 4 * hi;
                constexpr int H = C::DB / 2;
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    w[j] = pack_bf16x2(oacc[db][4 * g + j] * inv, oacc[db + H][4 * g + j] * inv);
                *(u32x4*)(op + 2 * p0) = u32x4{w[0], w[1], w[2], w[3]};
            }
        if (lse && hi == 0)
            lse[(size_t)bh * Tq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                               bool causal, float scale, hipStream_t stream) {
    const int BH = B * Hq;
    const int n_qtiles = (Tq + kBM - 1) / kBM;
    const dim3 grid(BH * n_qtiles);
    const float sl2 = scale * kLog2e;
    auto go = [&](auto kern) {
        kern<<<grid, kThreads, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k,
                                            (const uint16_t*)v, (uint16_t*)o, lse, BH, Hq, Hkv,
                                            Tq, Tk, n_qtiles, sl2, nullptr, nullptr, 0);
    };
    if (D == 64)
        causal ? go(prefill_bf16_kernel<64, true, false>) : go(prefill_bf16_kernel<64, false, false>);
    else
        causal ? go(prefill_bf16_kernel<128, true, false>) : go(prefill_bf16_kernel<128, false, false>);
    return hipGetLastError();
}

hipError_t launch_prefill_paged_bf16(const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* block_table, const int32_t* kv_lens,
                                     void* o, float* lse, int B, int Hq, int Hkv, int Tq, int D,
                                     int bt_stride, bool causal, float scale, hipStream_t stream) {
    const int BH = B * Hq;
    const int n_qtiles = (Tq + kBM - 1) / kBM;
    const dim3 grid(BH * n_qtiles);
    const float sl2 = scale * kLog2e;
    auto go = [&](auto kern) {
        kern<<<grid, kThreads, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k_pages,
                                            (const uint16_t*)v_pages, (uint16_t*)o, lse, BH, Hq,
                                            Hkv, Tq, 0, n_qtiles, sl2, block_table, kv_lens,
                                            bt_stride);
    };
    if (D == 64)
        causal ? go(prefill_bf16_kernel<64, true, true>) : go(prefill_bf16_kernel<64, false, true>);
    else
        causal ? go(prefill_bf16_kernel<128, true, true>) : go(prefill_bf16_kernel<128, false, true>);
    return hipGetLastError();
}

}  // namespace attn
