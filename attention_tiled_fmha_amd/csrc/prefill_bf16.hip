// Dense and paged prefill FMHA, bf16 in/out, on gfx950 bf16 MFMA with fp32
// accumulation.
//
// Method: the fused, tiled attention of the TensorRT-LLM FMHA page
// (zyxy.net/?p=24414, section 2: score, softmax and weighted sum fused in one
// kernel, tiles staged on chip, a bank-conflict-free on-chip layout, stable
// softmax) with the online softmax update of FlashAttention (FlashDecoding++
// summary, wenjunhu.com/d/2311396.html, section 1), so the T x T score matrix
// never leaves registers.  K/V tiles are double-buffered in LDS and the next
// ones are in flight from HBM while the current ones are consumed (the
// ping-pong buffering of the same summary, section 4).
//
// gfx950 mapping
// --------------
// A workgroup is 4 wavefronts, one per SIMD, and owns 128 query rows of one
// (batch, head); each wavefront holds one 32-row block of them.  Two
// workgroups share a CU (at most 256 registers per wavefront), so every
// SIMD runs two wavefronts of two independent workgroups: while one waits at
// its workgroup's barrier or for its loads, or runs its softmax on the VALU,
// the other issues MFMAs.  Per key tile of 32 keys a wavefront computes
//
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS, B = Q held in
//                   VGPRs.  S^T puts one query row per lane and 16 of the 32
//                   keys in its registers (the rest in lane l ^ 32): row max
//                   and row sum are lane-local plus one v_permlane32_swap.
//   softmax         exp2 of the scaled scores against a fixed per-row
//                   reference, P rounded to bf16, already in B-operand
//                   order for PV.
//   O^T += V^T P^T  A = V^T read from the row-major V tile with the gfx950
//                   transposing LDS read ds_read_b64_tr_b16.
//
// The three jobs of a step run interleaved in one instruction stream: step
// t issues the MFMAs of S(t+1) and of O += P(t-1) V(t-1) while the VALU runs
// the softmax of S(t).  kOne = false selects the earlier mapping (256-row
// tiles, two 32-row blocks per wavefront, blocks w and 7 - w, one workgroup
// per CU: every K/V fragment read from LDS feeds two blocks, but a barrier
// wait or an unhidden softmax leaves the SIMD idle); the single-block mapping
// gives bit-identical results and ran the causal prefill 4.3% faster, the
// non-causal 2.4% and the chunked prefill 5% in interleaved A/B runs.
//
// K/V tiles go from HBM straight into LDS (buffer loads with the LDS
// destination, no VGPR staging): step t issues the loads of its tile pair
// into the stage that step t - 1 finished reading, each wavefront waits for
// its own loads at the end of the step, and the step's workgroup barrier
// hands the tiles over.  Each stage is its own LDS object, so the compiler
// orders reads of one stage only after the loads into that stage.  LDS rows
// are 16-byte-granule XOR swizzled: the 16 rows one K read spans and the 4
// rows x 4 granules one transposed V read spans each hit 16 distinct granule
// positions of the 64 banks; a wavefront's load fills 1 KiB contiguously.
//
// Registers: the MFMAs write VGPRs (the library builds this file with the
// VGPR form of the matrix instructions), so the softmax reads S without
// copies, and the Q fragments, which only the S MFMAs read, are placed in
// AGPRs; a wavefront's block then needs about 200 registers (O, two sets of
// S, Q, P and the LDS reads issued several MFMAs ahead), within the 256 that
// two wavefronts per SIMD leave each (the two-block mapping used ~405 of 512
// at one wavefront per SIMD).
//
// Softmax reference.  Each row's exponentials are taken against the row max
// of its first key tile, held for the whole pass, so no running max is kept
// and O and l are never rescaled: numerator and denominator share the
// reference, which is exact in exact arithmetic.  A later key far above the
// reference would overflow, so every step checks that the tile's row sum
// stays <= 2^20; if any row of any wavefront exceeds it, the workgroup
// computes the exact row maxima over every visible key and runs the pass
// again against them (every P <= 1).  The row sum adds the bf16-rounded P
// that the MFMA multiplies with V.
//
// Causal masking (key j visible to query i iff j <= i + Tk - Tq) is applied
// only on tiles that cross a block's diagonal.  Once a wavefront's block is
// past its last visible key tile, its remaining steps only load and
// synchronise (two-block mapping: they run on the later block alone), which
// removes most of the work above the diagonal.  When there are at least two
// query tiles per workgroup slot (four per CU), a workgroup takes query
// tiles p and n - 1 - p of one (b, h) (equal causal work per workgroup), the
// heavier one first, and the workgroups of one
// (b, h) sit on one XCD at the same time: their heavier tiles walk the
// shared keys in step, so one fetch from HBM serves both through that XCD's
// L2.  The lighter tiles come later and fetch their keys again (an XCD's L2
// holds about the last 8 key tiles of its 32 workgroups).  Otherwise every
// workgroup takes one query tile, heaviest first.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

#define LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// single-block mode: one 32-row block per wavefront, 128-row query tiles,
// two workgroups per CU
constexpr bool kOne = true;
constexpr int kBM = kOne ? 128 : 256;    // query rows per query tile
constexpr int kBN = 32;                  // keys per K/V tile
constexpr float kRescaleThresh = 8.0f;   // log2 units

template <int D>
struct Cfg {
    static constexpr int KS = D / 16;              // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;              // 32-dim blocks of O^T
    static constexpr int GPR = D / 8;              // 16-byte granules per row
    static constexpr int ROW = 2 * D;              // bytes per K/V row
    static constexpr int TILE = kBN * ROW;         // bytes per K or V tile
    static constexpr int LPT = kBN * GPR / kThreads;  // 16-byte loads per thread per K or V tile
};

// The blocks each of a step's three jobs (S of the next key tile, softmax
// of the current one, PV of the previous one) covers: 2 both of the
// wavefront's row blocks, 1 only the later one (rb1), 0 none.
template <int S, int M, int V>
struct Jobs {
    static constexpr int s = S, m = M, v = V;
};

// Granule positions.  K (read 16 rows x one granule per instruction):
// D = 128 rows are 256 bytes, position c ^ (r mod 16); D = 64 rows are 128
// bytes (two per bank sweep), position c ^ (r/2 mod 8).  V (read 4 rows x 4
// granules per 32 lanes): D = 128 position c ^ 4(r mod 4); D = 64
// c ^ 4(r/2 mod 2).
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }

// Raw buffer resource over `bytes` bytes from base.  Loads at or past the
// size return zeros without touching memory, so tail tiles, tiles past the
// key range and pages past a sequence's length need no branch; the
// descriptor is built with scalar ALU only.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// Where the K/V of one (b, kv head) live: a dense [Tk][D] slice, or a
// sequence's block-table row over the paged pools [pages][Hkv][16][D].
struct KVSrc {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* table;   // paged: this sequence's block-table row
    int Hkv, kvh, Tk;
    unsigned* err;          // checked build: error word and pool size
    int num_pages;
};

// Thread tid's granules of a tile: g = tid + 256 j lands at byte 16 g of the
// LDS tile (row g / GPR, swizzled position g % GPR), so it fetches global
// granule (g % GPR) ^ swz(row) of that row.  goff is its byte offset within
// the tile (dense) or within its 16-row page (paged); a wavefront's load j
// covers rows of one page.
template <int D>
struct LoadPlan {
    int goff_k[Cfg<D>::LPT], goff_v[Cfg<D>::LPT];
    __device__ LoadPlan(int tid, bool paged) {
        using C = Cfg<D>;
#pragma unroll
        for (int j = 0; j < C::LPT; j++) {
            const int g = tid + kThreads * j, r = g / C::GPR, p = g % C::GPR;
            const int rr = paged ? (r & 15) : r;
            goff_k[j] = rr * C::ROW + 16 * (p ^ k_swz<D>(r));
            goff_v[j] = rr * C::ROW + 16 * (p ^ v_swz<D>(r));
        }
    }
};

// One 16-byte global -> LDS load per lane: lane L of the wavefront writes
// bytes dst + 16 L .. + 15 (the LDS address is the wavefront's M0 base).  A
// lane whose offset lies past the descriptor's size writes zeros.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char LDS_AS* dst,
                                           int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void LDS_AS*)dst, 16, off, 0, 0, 0);
}

// Issue this thread's direct-to-LDS loads of K tile kt into kdst and, with
// V_TOO, of V tile vt into vdst: granule j of thread tid lands at byte
// 16 (tid + 256 j) of the tile, i.e. wavefront w's load j fills the 1 KiB at
// 1024 (w + 4 j).  Tiles below 0 or past Tk are empty (zero-sized
// descriptors), so their LDS bytes become zeros and every call issues the
// same number of loads.
template <int D, bool PAGED, bool V_TOO>
__device__ __forceinline__ void dma_tiles(unsigned char LDS_AS* kdst, unsigned char LDS_AS* vdst,
                                          const KVSrc& src, const LoadPlan<D>& lp, int wave,
                                          int kt, int vt) {
    using C = Cfg<D>;
#pragma unroll
    for (int j = 0; j < C::LPT; j++) {
        const uint16_t* kb;
        const uint16_t* vb;
        int kbytes, vbytes;
        if constexpr (PAGED) {
            // rows of load j of this wavefront: one 16-token page of the tile
            const int slot = (kThreads * j + 64 * wave) / C::GPR / 16;
            auto page = [&](const uint16_t* pool, int t, const uint16_t*& base, int& bytes) {
                const int p = t * (kBN / 16) + slot;
                const int valid = t < 0 ? 0 : max(0, min(16, src.Tk - p * 16));
                base = pool;
                if (__builtin_amdgcn_readfirstlane(valid) > 0) {
                    const int phys = __builtin_amdgcn_readfirstlane(
                        checked_page(src.table[p], src.num_pages, src.err));
                    base = pool + ((size_t)phys * src.Hkv + src.kvh) * 16 * D;
                }
                bytes = valid * C::ROW;
            };
            page(src.k, kt, kb, kbytes);
            page(src.v, vt, vb, vbytes);
        } else {
            auto rows = [&](int t) { return t < 0 ? 0 : max(0, min(kBN, src.Tk - t * kBN)); };
            kb = src.k + (size_t)max(kt, 0) * kBN * D;
            vb = src.v + (size_t)max(vt, 0) * kBN * D;
            kbytes = rows(kt) * C::ROW;
            vbytes = rows(vt) * C::ROW;
        }
        const int dst = 1024 * (wave + 4 * j);
        lds_load16(rsrc(kb, kbytes), kdst + dst, lp.goff_k[j]);
        if constexpr (V_TOO) lds_load16(rsrc(vb, vbytes), vdst + dst, lp.goff_v[j]);
    }
}

__device__ __forceinline__ bf16x8 tr_read_pair(const unsigned char LDS_AS* p0,
                                               const unsigned char LDS_AS* p1) {
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)p0);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 LDS_AS*)p1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup barrier that also orders LDS: this wavefront's LDS accesses are
// complete and no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same after this wavefront's direct-to-LDS loads (and every other
// vector memory access it issued) have completed: after it, every
// wavefront's tiles are in LDS.
__device__ __forceinline__ void dma_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kOne ? 2 : 1, kOne ? 2 : 1)))
void prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                         float* __restrict__ lse, int BH, int Hq, int Hkv, int Tq, int Tk_dense,
                         int n_qtiles, int paired, float scale_log2,
                         const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ kv_lens, int bt_stride,
                         unsigned* err, int num_pages) {
    using C = Cfg<D>;
    // two K and two V stages, each its own LDS object: the compiler then
    // tracks the direct-to-LDS loads into one stage separately from reads of
    // the others (a shared object would make every LDS read wait for every
    // load in flight)
    __shared__ __attribute__((aligned(1024))) unsigned char k_st0[C::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char k_st1[C::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char v_st0[C::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char v_st1[C::TILE];
    __shared__ int flags[kWaves];
    unsigned char LDS_AS* const sK[2] = {(unsigned char LDS_AS*)k_st0, (unsigned char LDS_AS*)k_st1};
    unsigned char LDS_AS* const sV[2] = {(unsigned char LDS_AS*)v_st0, (unsigned char LDS_AS*)v_st1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar
    const int li = lane & 31, hi = lane >> 5;
    const int rb0 = wave, rb1 = kOne ? wave : 7 - wave;   // this wavefront's 32-row blocks

    // Workgroups are dealt to the 8 XCDs round-robin, so id % 8 picks the
    // XCD.  slot = id % BH: kv group kg = slot % (B * Hkv), head within the
    // group g = slot / (B * Hkv), so every query tile of every head that reads
    // one kv head's K/V lands on one XCD when BH and B * Hkv are multiples of
    // 8 (without grouped heads slot = b * Hq + h).  Paired: unit p = id / BH
    // holds query tiles p and n - 1 - p; otherwise query tile n - 1 - id / BH.
    const int id = blockIdx.x;
    const int slot = id % BH, unit = id / BH;
    const int KG = (BH / Hq) * Hkv;      // (batch, kv head) groups
    const int kg = slot % KG, g_in = slot / KG;
    const int b = kg / Hkv, kvh = kg % Hkv, h = kvh * (Hq / Hkv) + g_in;
    const int bh = b * Hq + h;
    // paged: the sequence's own key count (its chunk of Tq queries is its
    // last Tq positions, so the causal diagonal sits at kv_len - Tq), clamped
    // to what its block-table row can map so no page index leaves the row
    if constexpr (PAGED) {
        if (blockIdx.x < BH && threadIdx.x == 0) check_len(kv_lens[b], bt_stride * 16, err);
    }
    const int Tk = PAGED ? __builtin_amdgcn_readfirstlane(max(0, min(kv_lens[b], bt_stride * 16)))
                         : Tk_dense;
    const int diag = Tk - Tq;

    const uint16_t* qp = q + (size_t)bh * Tq * D;
    KVSrc src;
    src.k = PAGED ? k : k + (size_t)(b * Hkv + kvh) * Tk * D;
    src.v = PAGED ? v : v + (size_t)(b * Hkv + kvh) * Tk * D;
    src.table = PAGED ? block_table + (size_t)b * bt_stride : nullptr;
    src.Hkv = Hkv;
    src.kvh = kvh;
    src.Tk = Tk;
    src.err = err;
    src.num_pages = num_pages;
    const LoadPlan<D> lp(tid, PAGED);

    // Per-lane LDS offsets of the MFMA operands within a K or V tile.
    // K (A of S^T = K Q^T): row li, dims 16s + 8hi .. +7.  V^T (A of
    // O^T = V^T P^T) via transposing reads: within each 16-lane group g, lane
    // j addresses key row kbase + j/4 and 4 dims; lane i then holds dims d(i)
    // of keys kbase .. kbase + 3.  The dims are chosen so that O^T register r
    // of lane l is dim 32db + 16(r/8) + 8hi + r%8, which makes the epilogue's
    // stores 16 contiguous bytes.
    int koff[C::KS], voff[C::DB];
#pragma unroll
    for (int s = 0; s < C::KS; s++) koff[s] = li * C::ROW + 16 * ((2 * s + hi) ^ k_swz<D>(li));
    {
        const int g = lane >> 4, j = lane & 15;
        const int vx = D == 128 ? (j >> 2) : ((j >> 3) & 1);    // v_swz(row) / 4
#pragma unroll
        for (int db = 0; db < C::DB; db++)
            voff[db] = (4 * (g >> 1) + (j >> 2)) * C::ROW + 16 * (2 * (g & 1) + (j & 1)) +
                       64 * (db ^ vx) + 8 * ((j >> 1) & 1);
    }

    const int n_my = paired ? ((n_qtiles - 1 - unit) == unit ? 1 : 2) : 1;
    // the heavier tile of a pair first (the pairs of one (b, h) then share
    // their longest runs of key tiles)
    const int first = n_qtiles - 1 - unit;
    auto tile_of = [&](int u) {
        return paired ? (u == 0 ? first : n_qtiles - 1 - first) : n_qtiles - 1 - unit;
    };
    // Q fragments (B operand of S^T = K Q^T) of the current query tile: row
    // qrow, dims 16s + 8hi .. +7, loaded unconditionally (clamped row, zeroed
    // past Tq).  The first K tiles of a pass (K(0) and K(1), with zeros for
    // V stage 1) go to LDS ahead of it.
    bf16x8 qf[2][C::KS];
    auto issue_kv_head = [&]() {
        dma_tiles<D, PAGED, true>(sK[0], sV[1], src, lp, wave, 0, -1);
        dma_tiles<D, PAGED, false>(sK[1], sV[1], src, lp, wave, 1, -1);
    };
    auto issue_tile = [&](int u) {
        const int q0u = tile_of(u) * kBM;
#pragma unroll
        for (int a = kOne ? 1 : 0; a < 2; a++) {
            const int qrow = q0u + 32 * (a ? rb1 : rb0) + li;
            const int qr = min(qrow, max(Tq - 1, 0));
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                u32x4 w = *(const u32x4*)(qp + (size_t)qr * D + 16 * s + 8 * hi);
                if (qrow >= Tq) w = u32x4{0, 0, 0, 0};
                // an empty statement whose operand lives in AGPRs: Q stays
                // there, as the B operand of the S MFMAs
                asm("" : "+a"(w));
                qf[a][s] = __builtin_bit_cast(bf16x8, w);
            }
        }
        issue_kv_head();
    };
    issue_tile(0);
    for (int u = 0; u < n_my; u++) {
        const int qt = tile_of(u);
        const int q0 = qt * kBM;
        const int qa0 = q0 + 32 * rb0, qa1 = q0 + 32 * rb1;     // first rows of the blocks
        const int qrow0 = qa0 + li, qrow1 = qa1 + li;

        // key tiles of the query tile (the later block's range bounds both)
        const int kend = CAUSAL ? max(0, min(Tk, q0 + kBM + diag)) : Tk;
        const int n = (kend + kBN - 1) / kBN;
        // first tile that needs a mask for either block: the one holding key
        // Tk (partial tile) or, causal, the first key past the earlier block's
        // first row
        const int t_mask = CAUSAL ? max(0, min(Tk, (kOne ? qa1 : qa0) + diag + 1)) / kBN : Tk / kBN;
        // per-block last visible key of this lane's row
        const int lim0 = CAUSAL ? min(Tk - 1, qrow0 + diag) : Tk - 1;
        const int lim1 = CAUSAL ? min(Tk - 1, qrow1 + diag) : Tk - 1;

        f32x16 oacc[2][C::DB];
        float m_ref[2], l_run[2];
        f32x16 sacc[2][2];      // [parity][block]
        bf16x8 pf[2][2][2];     // [parity][block][16-key step]; pf[1] starts as P(-1) = 0

        // S^T(t) for both blocks from K tile t (LDS stage t % 2) into sacc[t % 2]
        auto s_mfma = [&](auto PAR) {
            constexpr int P = decltype(PAR)::value;
            const unsigned char LDS_AS* sk = sK[P];
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                const bf16x8 kf = *(const bf16x8 LDS_AS*)(sk + koff[s]);
#pragma unroll
                for (int a = kOne ? 1 : 0; a < 2; a++)
                    sacc[P][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        kf, qf[a][s], s == 0 ? f32x16{} : sacc[P][a], 0, 0, 0);
            }
        };
        // mask the scores of tile t: key k0 + 4hi + e (e = 8(r/4) + r%4) is
        // visible iff e <= the lane's last visible key - k0 - 4hi
        int t_cur = 0;   // tile whose scores the mask applies to
        auto mask_tile = [&](f32x16& x, int a) {
            const int lim = (a ? lim1 : lim0) - t_cur * kBN - 4 * hi;
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (8 * (r >> 2) + (r & 3) > lim) x[r] = -INFINITY;
        };
        auto row_max = [&](const f32x16& x) {
            float a0 = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), x[2]);
            float a1 = __builtin_fmaxf(__builtin_fmaxf(x[3], x[4]), x[5]);
            float a2 = __builtin_fmaxf(__builtin_fmaxf(x[6], x[7]), x[8]);
            float a3 = __builtin_fmaxf(__builtin_fmaxf(x[9], x[10]), x[11]);
            float a4 = __builtin_fmaxf(__builtin_fmaxf(x[12], x[13]), x[14]);
            a0 = __builtin_fmaxf(__builtin_fmaxf(a0, a1), a2);
            a3 = __builtin_fmaxf(__builtin_fmaxf(a3, a4), x[15]);
            const float m = half_swap_max(__builtin_fmaxf(a0, a3));
            return (m == -INFINITY) ? -INFINITY : m * scale_log2;
        };
        // One step as a fixed sequence of NS slots (a scheduling barrier after
        // each, so the compiler keeps the order): slot i issues one MFMA (S and
        // PV alternate, so each S MFMA's dependence on the previous one of its
        // chain is four slots back), one stage of the softmax (the fma of
        // score i, the exp2 of score i - 1, and every second slot the bf16 pack
        // and row sum of the pair before), and the LDS reads of the operands
        // needed LA slots later.  MFMA and VALU work share the SIMD's issue
        // capacity, so a steady mix keeps both busy.
        constexpr int NS = 4 * C::KS;       // MFMAs per step (2 KS for S, 2 KS for PV)
        constexpr int LA = 6;               // read lookahead in slots
        auto step_body = [&](auto PAR, auto MASK, auto FIRST, auto JOBS) -> bool {
            constexpr int P = decltype(PAR)::value, NP = P ^ 1;
            using J = decltype(JOBS);
            constexpr int SB = J::s, MB = J::m, VB = J::v;
            // the active scores: those of block 1 (16 .. 31), or of both
            constexpr int SC0 = 32 - 16 * MB, SCN = 16 * MB;
            const unsigned char LDS_AS* sk = sK[NP];
            const unsigned char LDS_AS* sv = sV[NP];
            bool big = false;
            float m_eff[2];
            int limt[2];   // masked steps: register r of block a is visible iff 8(r/4) + r%4 <= limt[a]
#pragma unroll
            for (int a = kOne ? 1 : 0; a < 2; a++) {
                limt[a] = (a ? lim1 : lim0) - t_cur * kBN - 4 * hi;
                if constexpr (decltype(FIRST)::value) {
                    mask_tile(sacc[P][a], a);
                    m_ref[a] = row_max(sacc[P][a]);
                }
                m_eff[a] = (m_ref[a] == -INFINITY) ? 0.f : m_ref[a];
            }
            // slot of the MFMA that first uses K fragment s / V fragment (ps, db)
            auto k_slot = [](int s2) { return 4 * s2; };
            auto v_slot = [](int ps, int db) { return 4 * (C::DB * ps + db) + 1; };
            bf16x8 kf[C::KS], vf[2][C::DB];
            auto read_k = [&](int s2) { kf[s2] = *(const bf16x8 LDS_AS*)(sk + koff[s2]); };
            auto read_v = [&](int ps, int db) {
                const unsigned char LDS_AS* a0 = sv + 16 * ps * C::ROW + voff[db];
                vf[ps][db] = tr_read_pair(a0, a0 + 8 * C::ROW);
            };
            // reads needed before slot LA
#pragma unroll
            for (int s2 = 0; s2 < C::KS; s2++)
                if (SB > 0 && k_slot(s2) < LA) read_k(s2);
#pragma unroll
            for (int ps = 0; ps < 2; ps++)
#pragma unroll
                for (int db = 0; db < C::DB; db++)
                    if (VB > 0 && v_slot(ps, db) < LA) read_v(ps, db);
            float pe[32];                      // exp2 results awaiting their pack
            float lsum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            uint32_t pw[2][2][4];
            auto sm_fma = [&](int j) {         // score j: block j / 16, register j % 16
                const int a = j >> 4, r = j & 15;
                const float y = __builtin_fmaf(sacc[P][a][r], scale_log2, -m_eff[a]);
                pe[j] = (decltype(MASK)::value && 8 * (r >> 2) + (r & 3) > limt[a]) ? -INFINITY : y;
            };
            auto sm_exp = [&](int j) { pe[j] = fast_exp2(pe[j]); };
            auto sm_pack = [&](int j) {        // pair (j, j + 1), j even
                const int a = j >> 4, r = j & 15, ps = r >> 3, e = (r & 7) >> 1;
                const uint32_t w = pack_bf16x2(pe[j], pe[j + 1]);
                pw[a][ps][e] = w;
                float& acc = lsum[a][e & 1];
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                                      __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
            };
#pragma unroll
            for (int i = 0; i < NS; i++) {
                if (i % 2 == 0) {   // S MFMA: k-step s of block a
                    const int s2 = i / 4, a = (i / 2) % 2;
                    if (a >= 2 - SB)
                        sacc[NP][a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            kf[s2], qf[a][s2], s2 == 0 ? f32x16{} : sacc[NP][a], 0, 0, 0);
                } else {            // PV MFMA: 16-key step ps, dim block db, block a
                    const int k2 = i / 2, ps = k2 / (2 * C::DB), db = (k2 / 2) % C::DB, a = k2 % 2;
                    if (a >= 2 - VB)
                        oacc[a][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vf[ps][db], pf[NP][a][ps], oacc[a][db], 0, 0, 0);
                }
                // the active scores spread evenly over the slots
#pragma unroll
                for (int j = SC0 + i * SCN / NS; j < SC0 + (i + 1) * SCN / NS; j++) {
                    sm_fma(j);
                    if (j - 1 >= SC0) sm_exp(j - 1);
                    if (j - 3 >= SC0 && (j & 1)) sm_pack(j - 3);
                }
#pragma unroll
                for (int s2 = 0; s2 < C::KS; s2++)
                    if (SB > 0 && k_slot(s2) == i + LA) read_k(s2);
#pragma unroll
                for (int ps = 0; ps < 2; ps++)
#pragma unroll
                    for (int db = 0; db < C::DB; db++)
                        if (VB > 0 && v_slot(ps, db) == i + LA) read_v(ps, db);
            }
            __builtin_amdgcn_iglp_opt(3);
            if constexpr (MB > 0) {
                // the slots packed pairs up to 28; pair 30 remains
                sm_exp(31);
                sm_pack(30);
            }
#pragma unroll
            for (int a = 2 - MB; a < 2; a++) {
#pragma unroll
                for (int ps = 0; ps < 2; ps++)
                    pf[P][a][ps] = __builtin_bit_cast(bf16x8, u32x4{pw[a][ps][0], pw[a][ps][1],
                                                                   pw[a][ps][2], pw[a][ps][3]});
                const float lt = lsum[a][0] + lsum[a][1];
                l_run[a] += lt;
                big |= !(lt <= 1048576.f);   // also catches inf and NaN sums
            }
            return __builtin_amdgcn_ballot_w64(big) != 0;
        };

        // last key tile of this wavefront's block 0 (the one that holds the
        // last key its last row sees; -1 when it sees none)
        const int qaT = kOne ? qa1 : qa0;
        const int T0 = CAUSAL ? (min(Tk - 1, qaT + 31 + diag) >= 0 ? min(Tk - 1, qaT + 31 + diag) / kBN : -1)
                              : n - 1;
        // One pass over the key tiles.  Step t: S(t+1), softmax(t), PV(t-1);
        // pair t (K(t+2), V(t)) is loaded into LDS stage t%2, which step t - 1
        // was the last to read; S(t+1) and PV(t-1) read stage (t+1)%2.  Every
        // step runs all three jobs: PV(-1) multiplies P = 0 with the zeroed V
        // stage 1, S(n) and S(n+1) read tiles past the key range (zeros) and
        // are not used, and the softmax of step n sees only masked keys (P = 0).
        // Steps from t_mask on apply the mask.  GIVEN: m_ref holds the exact
        // row maxima (the recompute pass), else it is taken from tile 0.
        // Returns whether any wavefront saw a too-low reference.
        auto pass = [&](auto GIVEN) -> bool {
            constexpr bool G = decltype(GIVEN)::value;
            const std::integral_constant<bool, true> Y;
            const std::integral_constant<bool, false> N;
            const std::integral_constant<int, 0> P0;
            const std::integral_constant<int, 1> P1;
#pragma unroll
            for (int a = 0; a < 2; a++) {
                l_run[a] = 0.f;
#pragma unroll
                for (int db = 0; db < C::DB; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[a][db][r] = 0.f;
#pragma unroll
                for (int ps = 0; ps < 2; ps++) pf[1][a][ps] = bf16x8{};
            }
            bool flag = false;
            auto step = [&](int t, auto PAR, auto MASK, auto FIRST, auto JOBS) {
                constexpr int P = decltype(PAR)::value;          // t % 2
                dma_tiles<D, PAGED, true>(sK[P], sV[P], src, lp, wave, t + 2, t);
                // the loads go out first: they have the whole step to land
                __builtin_amdgcn_sched_barrier(0);
                t_cur = t;
                const bool big = step_body(PAR, MASK, FIRST, JOBS);
                if constexpr (!G) flag |= big;
                dma_barrier();
            };
            // prologue (its loads were issued ahead): K(0) and K(1) in LDS,
            // zeros in V stage 1; then S(0)
            dma_barrier();
            s_mfma(P0);
            lds_barrier();                    // K stage 0 is rewritten in step 0
            // Step 0 (masked, which is exact for any tile), then pairs of steps
            // (t odd, t + 1) so that the register sets keep their roles:
            // unmasked pairs while both steps precede t_mask, then masked pairs
            // up to step n (masking a tile that needs none, or running a step
            // past n, changes nothing).
            using BothJ = std::conditional_t<kOne, Jobs<1, 1, 1>, Jobs<2, 2, 2>>;
            const BothJ BOTH;
            step(0, P0, Y, std::integral_constant<bool, !G>{}, BOTH);
            int t = 1;
            for (; t + 2 <= t_mask; t += 2) {
                step(t, P1, N, N, BOTH);
                step(t + 1, P0, N, N, BOTH);
            }
            // causal: once block 0 is past its last key tile T0 (from step
            // T0 + 2 on it has no S, softmax or PV left), the pairs run on
            // block 1 alone
            const int t_half = CAUSAL ? T0 + 2 : n + 2;
            for (; t <= n && t < t_half; t += 2) {
                step(t, P1, Y, N, BOTH);
                step(t + 1, P0, Y, N, BOTH);
            }
            if constexpr (CAUSAL) {
                // single-block mode: past its block's last key tile a
                // wavefront only loads and synchronises
                using HalfJ = std::conditional_t<kOne, Jobs<0, 0, 0>, Jobs<1, 1, 1>>;
                for (; t <= n; t += 2) {
                    step(t, P1, Y, N, HalfJ{});
                    step(t + 1, P0, Y, N, HalfJ{});
                }
            }
            return flag;
        };

        if (n > 0) {
            bool flag = pass(std::integral_constant<bool, false>{});
            // any wavefront's flag makes the whole workgroup recompute
            if (lane == 0) flags[wave] = flag;
            lds_barrier();
            flag = flags[0] | flags[1] | flags[2] | flags[3];
            lds_barrier();
            if (flag) {
                // exact row maxima over every visible key, then the same pass
                // against them (every P <= 1)
                m_ref[0] = m_ref[1] = -INFINITY;
                for (int t = 0; t < n; t++) {
                    dma_tiles<D, PAGED, false>(sK[0], sV[1], src, lp, wave, t, -1);
                    dma_barrier();
                    s_mfma(std::integral_constant<int, 0>{});
#pragma unroll
                    for (int a = kOne ? 1 : 0; a < 2; a++) {
                        t_cur = t;
                        mask_tile(sacc[0][a], a);
                        m_ref[a] = fmaxf(m_ref[a], row_max(sacc[0][a]));
                    }
                    lds_barrier();
                }
                issue_kv_head();
                pass(std::integral_constant<bool, true>{});
            }
        } else {
            m_ref[0] = m_ref[1] = -INFINITY;
            l_run[0] = l_run[1] = 0.f;
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int db = 0; db < C::DB; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[a][db][r] = 0.f;
        }

        // the next query tile's Q and first K/V tiles load during this epilogue
        if (u + 1 < n_my) issue_tile(u + 1);

        // ---- epilogue: O = O / l, lse = m ln2 + ln l ------------------------
#pragma unroll
        for (int a = kOne ? 1 : 0; a < 2; a++) {
            const int qrow = a ? qrow1 : qrow0;
            const float l_tot = half_swap_sum(l_run[a]);
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (qrow < Tq) {
                uint16_t* op = o + ((size_t)bh * Tq + qrow) * D;
#pragma unroll
                for (int db = 0; db < C::DB; db++)
#pragma unroll
                    for (int jj = 0; jj < 2; jj++) {
                        uint32_t w[4];
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            w[e] = pack_bf16x2(oacc[a][db][8 * jj + 2 * e] * inv,
                                               oacc[a][db][8 * jj + 2 * e + 1] * inv);
                        *(u32x4*)(op + 32 * db + 16 * jj + 8 * hi) = u32x4{w[0], w[1], w[2], w[3]};
                    }
                if (lse && hi == 0)
                    lse[(size_t)bh * Tq + qrow] =
                        l_tot > 0.f ? (m_ref[a] + __log2f(l_tot)) * kLn2 : -INFINITY;
            }
        }
        // the next query tile's prologue rewrites every stage
        lds_barrier();
    }
}

// Pair query tiles p and n - 1 - p in one workgroup when that still leaves
// at least one workgroup per CU.
void grid_of(int BH, int n_qtiles, dim3* grid, int* paired) {
    // pairs only while they still leave kOne ? 2 : 1 workgroups per CU
    *paired = (long)BH * n_qtiles >= (kOne ? 4L : 2L) * device_cus() && n_qtiles >= 2;
    *grid = dim3(BH * (*paired ? (n_qtiles + 1) / 2 : n_qtiles));
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                               bool causal, float scale, hipStream_t stream) {
    const int BH = B * Hq;
    const int n_qtiles = (Tq + kBM - 1) / kBM;
    dim3 grid;
    int paired;
    grid_of(BH, n_qtiles, &grid, &paired);
    const float sl2 = scale * kLog2e;
    auto go = [&](auto kern) {
        kern<<<grid, kThreads, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k,
                                            (const uint16_t*)v, (uint16_t*)o, lse, BH, Hq, Hkv,
                                            Tq, Tk, n_qtiles, paired, sl2, nullptr, nullptr, 0,
                                            nullptr, 0);
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
                                     int bt_stride, bool causal, float scale, hipStream_t stream,
                                     unsigned* err, int num_pages) {
    const int BH = B * Hq;
    const int n_qtiles = (Tq + kBM - 1) / kBM;
    dim3 grid;
    int paired;
    grid_of(BH, n_qtiles, &grid, &paired);
    const float sl2 = scale * kLog2e;
    auto go = [&](auto kern) {
        kern<<<grid, kThreads, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k_pages,
                                            (const uint16_t*)v_pages, (uint16_t*)o, lse, BH, Hq,
                                            Hkv, Tq, 0, n_qtiles, paired, sl2, block_table, kv_lens,
                                            bt_stride, err, num_pages);
    };
    if (D == 64)
        causal ? go(prefill_bf16_kernel<64, true, true>) : go(prefill_bf16_kernel<64, false, true>);
    else
        causal ? go(prefill_bf16_kernel<128, true, true>) : go(prefill_bf16_kernel<128, false, true>);
    return hipGetLastError();
}

}  // namespace attn
