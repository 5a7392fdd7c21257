// Dense prefill FMHA, bf16 in/out, on gfx950 bf16 MFMA with fp32 accumulation.
//
// Method: the fused, tiled attention of the TensorRT-LLM FMHA page
// (zyxy.net/?p=24414, section 2: score, softmax and weighted sum fused in one
// kernel, tiles staged on chip, bank-conflict-aware on-chip layout, stable
// softmax) with the online softmax update of FlashAttention (FlashDecoding++
// summary, wenjunhu.com/d/2311396.html, section 1), so the T x T score matrix
// never leaves registers.  K/V tiles are double-buffered in LDS: the next
// tile is fetched while the current one is consumed (the ping-pong buffer of
// the same summary, section 4).
//
// gfx950 mapping
// --------------
// Workgroup = 4 wavefronts (one per SIMD) = BM = 256 query rows of one
// (batch, head); each wavefront owns 64 rows as two 32-row blocks.  Per key
// tile of BN = 32 keys:
//
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K from LDS (row-major),
//                   B = Q held in VGPRs for the whole kernel.
//   softmax         the accumulator of S^T gives lane l the scores of query
//                   row (l % 32) for 16 of the 32 keys; the other 16 are in
//                   lane l ^ 32.  Row max / sum are lane-local plus one
//                   permlane32 swap -- no LDS, no cross-row shuffles.
//   O^T += V^T P^T  A = V^T from LDS (V is transposed while it is written to
//                   LDS), B = P: the S^T accumulator registers, rounded to
//                   bf16, already sit in B-operand order.
//
// The running max is only raised (and O, l rescaled) when a row's max grows
// by more than 2^8; otherwise exponentials are taken against the stale max.
// Results are identical in exact arithmetic (numerator and denominator share
// the same reference), and every exponential stays <= 2^8, so nothing
// overflows in fp32.  The row sum l adds up the bf16-rounded P that the MFMA
// multiplies with V, so numerator and denominator see the same weights.
//
// Causal masking (key j visible to query i iff j <= i + Tk - Tq) costs only
// on tiles that cross the diagonal; tiles wholly above it are skipped per
// wavefront.  Workgroups are issued heaviest (longest key range) first, and
// all query tiles of one (b, h) land on one XCD so K/V reuse stays in its L2.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kWaves = 4;
constexpr int kIB = 2;                      // 32-row blocks per wavefront
constexpr int kBM = kWaves * kIB * 32;      // 256 query rows per workgroup
constexpr int kBN = 32;                     // keys per tile
constexpr float kRescaleThresh = 8.0f;      // log2 units

template <int D>
struct Cfg {
    static constexpr int KS = D / 16;             // MFMA k-steps of Q K^T
    static constexpr int DB = D / 32;             // 32-wide column blocks of O^T
    static constexpr int PS = kBN / 16;           // MFMA k-steps of P V
    static constexpr int KST = D + 8;             // K row stride in LDS (bf16)
    static constexpr int VST = kBN + 4;           // V^T row stride in LDS (bf16)
    static constexpr int K_ELEMS = kBN * KST;
    static constexpr int V_ELEMS = D * VST;
    // global -> register staging of one tile
    static constexpr int K_CHUNKS = D / 8;                      // 16-byte chunks per key row
    static constexpr int K_PASSES = kBN * K_CHUNKS / 256;       // 16-byte loads per lane
    static constexpr int V_UNITS = (kBN / 4) * (D / 4);         // 4 keys x 4 dims units
};

template <int D>
struct TileRegs {
    u32x4 k[Cfg<D>::K_PASSES];
    u32x2 v[4];
};

// Fetch one K/V tile (keys k0 .. k0+kBN-1) into registers; rows >= Tk are 0.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, int k0, int Tk,
                                          int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < C::K_PASSES; i++) {
        const int e = tid + 256 * i;
        const int row = e / C::K_CHUNKS, ch = e % C::K_CHUNKS;
        t.k[i] = (k0 + row < Tk) ? *(const u32x4*)(kp + (size_t)(k0 + row) * D + 8 * ch)
                                 : u32x4{0, 0, 0, 0};
    }
    if (tid < C::V_UNITS) {
        const int dg = tid % (D / 4), kg = tid / (D / 4);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int row = k0 + 4 * kg + j;
            t.v[j] = (row < Tk) ? *(const u32x2*)(vp + (size_t)row * D + 4 * dg) : u32x2{0, 0};
        }
    }
}

// Write a staged tile to LDS: K row-major, V transposed (V^T[d][key]).
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, uint16_t* sK, uint16_t* sV,
                                           int tid) {
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < C::K_PASSES; i++) {
        const int e = tid + 256 * i;
        const int row = e / C::K_CHUNKS, ch = e % C::K_CHUNKS;
        *(u32x4*)(sK + row * C::KST + 8 * ch) = t.k[i];
    }
    if (tid < C::V_UNITS) {
        const int dg = tid % (D / 4), kg = tid / (D / 4);
        // t.v[j] holds dims 4dg..4dg+3 of key 4kg+j; V^T[d][4kg..4kg+3] per dim
        u32x2 tr[4];
        transpose4x4_bf16(t.v, tr);
#pragma unroll
        for (int i = 0; i < 4; i++) *(u32x2*)(sV + (4 * dg + i) * C::VST + 4 * kg) = tr[i];
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                         float* __restrict__ lse, int BH, int Hq, int Hkv, int Tq, int Tk,
                         int n_qtiles, float scale_log2) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][C::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][C::V_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, hi = lane >> 5;

    // Heaviest query tiles first; bh = id % BH keeps one (b, h) on one XCD
    // when BH is a multiple of 8 (workgroups are dealt to XCDs round-robin).
    const int id = blockIdx.x;
    const int bh = id % BH;
    const int qt = n_qtiles - 1 - id / BH;
    const int b = bh / Hq, h = bh % Hq, kvh = h / (Hq / Hkv);
    const int q0 = qt * kBM;
    const int qw0 = q0 + wave * (kIB * 32);  // first row of this wavefront
    const int diag = Tk - Tq;

    const uint16_t* qp = q + (size_t)bh * Tq * D;
    const uint16_t* kp = k + (size_t)(b * Hkv + kvh) * Tk * D;
    const uint16_t* vp = v + (size_t)(b * Hkv + kvh) * Tk * D;

    // Q fragments (B operand of S^T = K Q^T): row li of each block, dims
    // 16s + 8hi .. +7.
    bf16x8 qf[kIB][C::KS];
#pragma unroll
    for (int ib = 0; ib < kIB; ib++) {
        const int row = qw0 + ib * 32 + li;
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            u32x4 w = (row < Tq) ? *(const u32x4*)(qp + (size_t)row * D + 16 * s + 8 * hi)
                                 : u32x4{0, 0, 0, 0};
            qf[ib][s] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Key range of the workgroup and of this wavefront.
    int kend = Tk;
    if (CAUSAL) kend = max(0, min(Tk, q0 + kBM + diag));
    int kend_w = Tk;
    if (CAUSAL) kend_w = max(0, min(Tk, qw0 + kIB * 32 + diag));
    const int n_tiles = (kend + kBN - 1) / kBN;

    f32x16 oacc[kIB][C::DB];
#pragma unroll
    for (int ib = 0; ib < kIB; ib++)
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) oacc[ib][db][r] = 0.f;
    float m_run[kIB], l_run[kIB];
#pragma unroll
    for (int ib = 0; ib < kIB; ib++) {
        m_run[ib] = -INFINITY;
        l_run[ib] = 0.f;
    }

    TileRegs<D> stage;
    if (n_tiles > 0) {
        load_tile<D>(stage, kp, vp, 0, Tk, tid);
        store_tile<D>(stage, sK[0], sV[0], tid);
    }
    __syncthreads();

    for (int kt = 0; kt < n_tiles; kt++) {
        const int buf = kt & 1;
        const int k0 = kt * kBN;
        if (kt + 1 < n_tiles) load_tile<D>(stage, kp, vp, k0 + kBN, Tk, tid);

        if (k0 < kend_w) {  // wavefront-uniform: some key of the tile is visible
            const uint16_t* tK = sK[buf];
            const uint16_t* tV = sV[buf];
            // ---- S^T = K Q^T ------------------------------------------------
            f32x16 sacc[kIB];
#pragma unroll
            for (int ib = 0; ib < kIB; ib++)
#pragma unroll
                for (int r = 0; r < 16; r++) sacc[ib][r] = 0.f;
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                const bf16x8 kf = *(const bf16x8*)(tK + li * C::KST + 16 * s + 8 * hi);
#pragma unroll
                for (int ib = 0; ib < kIB; ib++)
                    sacc[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ib][s], sacc[ib],
                                                                       0, 0, 0);
            }
            // ---- mask, online softmax ----------------------------------------
            // sacc[ib][r] is the score of key k0 + 8(r/4) + 4hi + r%4 for
            // query row qw0 + 32ib + li.
            const bool need_mask = (k0 + kBN > Tk) || (CAUSAL && k0 + kBN - 1 > qw0 + diag);
            bf16x8 pf[kIB][C::PS];
#pragma unroll
            for (int ib = 0; ib < kIB; ib++) {
                if (need_mask) {
                    const int qi = qw0 + ib * 32 + li;
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int kj = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        const bool vis = kj < Tk && (!CAUSAL || kj <= qi + diag);
                        if (!vis) sacc[ib][r] = -INFINITY;
                    }
                }
                float mx = sacc[ib][0];
#pragma unroll
                for (int r = 1; r < 16; r++) mx = fmaxf(mx, sacc[ib][r]);
                mx = half_swap_max(mx) * scale_log2;
                const float m_new = fmaxf(m_run[ib], mx);
                if (__builtin_amdgcn_ballot_w64(m_new > m_run[ib] + kRescaleThresh)) {
                    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[ib] - m_new);
                    l_run[ib] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::DB; db++) oacc[ib][db] *= alpha;
                    m_run[ib] = m_new;
                }
                const float m_eff = (m_run[ib] == -INFINITY) ? 0.f : m_run[ib];
#pragma unroll
                for (int ps = 0; ps < C::PS; ps++) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float p0 = fast_exp2(__builtin_fmaf(sacc[ib][8 * ps + 2 * e], scale_log2, -m_eff));
                        const float p1 = fast_exp2(__builtin_fmaf(sacc[ib][8 * ps + 2 * e + 1], scale_log2, -m_eff));
                        w[e] = pack_bf16x2(p0, p1);
                        l_run[ib] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2, w[e]),
                            __builtin_bit_cast(bf16x2, 0x3f803f80u), l_run[ib], false);
                    }
                    pf[ib][ps] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
            }
            // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
            for (int ps = 0; ps < C::PS; ps++) {
#pragma unroll
                for (int db = 0; db < C::DB; db++) {
                    const uint16_t* vrow = tV + (32 * db + li) * C::VST + 16 * ps + 4 * hi;
                    const u32x2 lo = *(const u32x2*)(vrow);
                    const u32x2 hi8 = *(const u32x2*)(vrow + 8);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi8[0], hi8[1]});
#pragma unroll
                    for (int ib = 0; ib < kIB; ib++)
                        oacc[ib][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ib][ps],
                                                                               oacc[ib][db], 0, 0, 0);
                }
            }
        }

        if (kt + 1 < n_tiles) store_tile<D>(stage, sK[buf ^ 1], sV[buf ^ 1], tid);
        __syncthreads();
    }

    // ---- epilogue: O = O / l, lse = m ln2 + ln l ----------------------------
#pragma unroll
    for (int ib = 0; ib < kIB; ib++) {
        const int row = qw0 + ib * 32 + li;
        const float l_tot = half_swap_sum(l_run[ib]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (row < Tq) {
            uint16_t* op = o + ((size_t)bh * Tq + row) * D;
#pragma unroll
            for (int db = 0; db < C::DB; db++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int d0 = 32 * db + 8 * g + 4 * hi;
                    *(u32x2*)(op + d0) = u32x2{
                        pack_bf16x2(oacc[ib][db][4 * g] * inv, oacc[ib][db][4 * g + 1] * inv),
                        pack_bf16x2(oacc[ib][db][4 * g + 2] * inv, oacc[ib][db][4 * g + 3] * inv)};
                }
            if (lse && hi == 0)
                lse[(size_t)bh * Tq + row] =
                    l_tot > 0.f ? (m_run[ib] + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
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
        kern<<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k,
                                       (const uint16_t*)v, (uint16_t*)o, lse, BH, Hq, Hkv, Tq,
                                       Tk, n_qtiles, sl2);
    };
    if (D == 64)
        causal ? go(prefill_bf16_kernel<64, true>) : go(prefill_bf16_kernel<64, false>);
    else
        causal ? go(prefill_bf16_kernel<128, true>) : go(prefill_bf16_kernel<128, false>);
    return hipGetLastError();
}

}  // namespace attn
