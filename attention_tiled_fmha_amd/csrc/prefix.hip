// Shared-prefix (cascade stage one) decode attention on bf16 MFMA.
//
// Every request attends the same prefix, stored once in the paged cache
// (prefix sharing of KV blocks, xhh.club summary, "how does paged attention
// manage the KV cache"; the staged cascade of "FlashInfer kernel library",
// sections 2 and 4).  For one kv head the R requests x G grouped heads form a
// block of query rows that all meet the same keys, so the prefix stage is a
// small dense attention, [R*G rows] x [prefix keys], and each prefix page is
// read from HBM exactly once per kv head for all requests -- instead of once
// per request, as R separate decodes would.
//
// gfx950 mapping: a workgroup (4 wavefronts) takes one kv head, a block of
// up to 64 query rows and one chunk of the prefix; each wavefront walks its
// own 32-key tiles of the chunk (two pages each), staging them through a
// private LDS region (K row-major, V transposed) while the next tile's loads
// are in flight:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q in VGPRs)
//   softmax       lane-local row statistics + one permlane32 swap
//   O^T += V^T P^T
// The four wavefront states are merged in LDS; the chunk's state goes to the
// workspace (or straight to the output when the prefix is one chunk), and
// the decode combine kernel folds the chunks with log-sum-exp.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int kPage = 16;
constexpr int kTile = 32;          // keys per wavefront tile (two pages)
constexpr float kRescaleThresh = 8.0f;

template <int D>
struct PCfg {
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int CPR = D / 8;              // 16-byte chunks per key row
    static constexpr int RPI = kWave / CPR;        // K rows per load instruction
    static constexpr int KLD = kTile / RPI;        // K loads per lane per tile
    static constexpr int VU = (kTile / 4) * CPR / kWave;  // 4-key x 8-dim units per lane
    static constexpr int KST = D + 8;
    static constexpr int VST = kTile + 4;
    static constexpr int WAVE_LDS = (kTile * KST + D * VST) * 2;  // bytes per wavefront
};

template <int D>
struct PTile {
    u32x4 k[PCfg<D>::KLD];
    u32x4 v[PCfg<D>::VU][4];
};

// Load the 32-key tile starting at key k0 of the prefix (keys >= L read as 0).
template <int D>
__device__ __forceinline__ void load_ptile(PTile<D>& t, const PrefixArgs& a, int kvh, int k0,
                                           int lane) {
    using C = PCfg<D>;
    const uint16_t* kp = (const uint16_t*)a.k_pages;
    const uint16_t* vp = (const uint16_t*)a.v_pages;
    const size_t page_elems = (size_t)a.Hkv * kPage * D;
    const size_t head_off = (size_t)kvh * kPage * D;
#pragma unroll
    for (int i = 0; i < C::KLD; i++) {
        const int row = i * C::RPI + lane / C::CPR, ch = lane % C::CPR;
        const int key = k0 + row;
        t.k[i] = u32x4{0, 0, 0, 0};
        if (key < a.prefix_len) {
            const size_t base = (size_t)a.pages[key / kPage] * page_elems + head_off;
            t.k[i] = *(const u32x4*)(kp + base + (size_t)(key % kPage) * D + 8 * ch);
        }
    }
#pragma unroll
    for (int u = 0; u < C::VU; u++) {
        const int unit = lane + kWave * u;
        const int dc = unit % C::CPR, kg = unit / C::CPR;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int key = k0 + 4 * kg + j;
            t.v[u][j] = u32x4{0, 0, 0, 0};
            if (key < a.prefix_len) {
                const size_t base = (size_t)a.pages[key / kPage] * page_elems + head_off;
                t.v[u][j] = *(const u32x4*)(vp + base + (size_t)(key % kPage) * D + 8 * dc);
            }
        }
    }
}

template <int D>
__device__ __forceinline__ void store_ptile(const PTile<D>& t, uint16_t* sK, uint16_t* sV,
                                            int lane) {
    using C = PCfg<D>;
#pragma unroll
    for (int i = 0; i < C::KLD; i++) {
        const int row = i * C::RPI + lane / C::CPR, ch = lane % C::CPR;
        *(u32x4*)(sK + row * C::KST + 8 * ch) = t.k[i];
    }
#pragma unroll
    for (int u = 0; u < C::VU; u++) {
        const int unit = lane + kWave * u;
        const int dc = unit % C::CPR, kg = unit / C::CPR;
#pragma unroll
        for (int half = 0; half < 2; half++) {   // dims 8dc + 4half .. +3
            const u32x2 rows[4] = {u32x2{t.v[u][0][2 * half], t.v[u][0][2 * half + 1]},
                                   u32x2{t.v[u][1][2 * half], t.v[u][1][2 * half + 1]},
                                   u32x2{t.v[u][2][2 * half], t.v[u][2][2 * half + 1]},
                                   u32x2{t.v[u][3][2 * half], t.v[u][3][2 * half + 1]}};
            u32x2 tr[4];
            transpose4x4_bf16(rows, tr);
#pragma unroll
            for (int i = 0; i < 4; i++)
                *(u32x2*)(sV + (8 * dc + 4 * half + i) * C::VST + 4 * kg) = tr[i];
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefix_kernel(PrefixArgs a) {
    using C = PCfg<D>;
    constexpr int IB = 2;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, hi = lane >> 5;
    const int c = blockIdx.x, kvh = blockIdx.y, rb = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const int N = a.R * G;  // query rows of this kv head
    const float sl2 = a.scale * kLog2e;

    uint16_t* sK = (uint16_t*)(smem + wave * C::WAVE_LDS);
    uint16_t* sV = sK + kTile * C::KST;

    // query rows n = rb*64 + 32ib + li: request n / G, head kvh*G + n % G
    const uint16_t* q = (const uint16_t*)a.q;
    bf16x8 qf[IB][C::KS];
#pragma unroll
    for (int ib = 0; ib < IB; ib++) {
        const int n = rb * 64 + ib * 32 + li;
        const size_t qrow = (size_t)(n / G) * a.Hq + kvh * G + n % G;
#pragma unroll
        for (int s = 0; s < C::KS; s++) {
            u32x4 w = (n < N) ? *(const u32x4*)(q + qrow * D + 16 * s + 8 * hi) : u32x4{0, 0, 0, 0};
            qf[ib][s] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x16 oacc[IB][C::DB];
#pragma unroll
    for (int ib = 0; ib < IB; ib++)
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) oacc[ib][db][r] = 0.f;
    float m_run[IB] = {-INFINITY, -INFINITY}, l_run[IB] = {0.f, 0.f};

    // this wavefront's tiles: keys c*chunk + (4t + wave)*32, t = 0 .. tiles_per_wave-1
    const int chunk0 = c * a.chunk;
    PTile<D> tile;
    load_ptile<D>(tile, a, kvh, chunk0 + wave * kTile, lane);
    for (int t = 0; t < a.tiles_per_wave; t++) {
        const int k0 = chunk0 + (4 * t + wave) * kTile;
        store_ptile<D>(tile, sK, sV, lane);
        __syncthreads();
        if (t + 1 < a.tiles_per_wave) load_ptile<D>(tile, a, kvh, k0 + 4 * kTile, lane);
        if (k0 < a.prefix_len) {
            f32x16 sacc[IB];
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int r = 0; r < 16; r++) sacc[ib][r] = 0.f;
#pragma unroll
            for (int s = 0; s < C::KS; s++) {
                const bf16x8 kf = *(const bf16x8*)(sK + li * C::KST + 16 * s + 8 * hi);
#pragma unroll
                for (int ib = 0; ib < IB; ib++)
                    sacc[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ib][s], sacc[ib], 0, 0, 0);
            }
            const bool tail = k0 + kTile > a.prefix_len;
            bf16x8 pf[IB][2];
#pragma unroll
            for (int ib = 0; ib < IB; ib++) {
                if (tail) {
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        if (k0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= a.prefix_len) sacc[ib][r] = -INFINITY;
                }
                float mx = sacc[ib][0];
#pragma unroll
                for (int r = 1; r < 16; r++) mx = fmaxf(mx, sacc[ib][r]);
                mx = half_swap_max(mx);
                mx = (mx == -INFINITY) ? -INFINITY : mx * sl2;
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
                for (int ps = 0; ps < 2; ps++) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float s0 = sacc[ib][8 * ps + 2 * e], s1 = sacc[ib][8 * ps + 2 * e + 1];
                        const float p0 = s0 == -INFINITY ? 0.f : fast_exp2(__builtin_fmaf(s0, sl2, -m_eff));
                        const float p1 = s1 == -INFINITY ? 0.f : fast_exp2(__builtin_fmaf(s1, sl2, -m_eff));
                        w[e] = pack_bf16x2(p0, p1);
                        l_run[ib] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2, w[e]), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                            l_run[ib], false);
                    }
                    pf[ib][ps] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
            }
#pragma unroll
            for (int ps = 0; ps < 2; ps++)
#pragma unroll
                for (int db = 0; db < C::DB; db++) {
                    const uint16_t* vrow = sV + (32 * db + li) * C::VST + 16 * ps + 4 * hi;
                    const u32x2 lo = *(const u32x2*)vrow;
                    const u32x2 hi8 = *(const u32x2*)(vrow + 8);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi8[0], hi8[1]});
#pragma unroll
                    for (int ib = 0; ib < IB; ib++)
                        oacc[ib][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ib][ps], oacc[ib][db], 0, 0, 0);
                }
        }
        __syncthreads();
    }

    // ---- merge the 4 wavefront states: (2,3) into (0,1), then 1 into 0 ----
    float l_tot[IB];
#pragma unroll
    for (int ib = 0; ib < IB; ib++) l_tot[ib] = half_swap_sum(l_run[ib]);
    float* xo = (float*)smem;                       // [2][IB*DB*16][64]
    float* xm = xo + 2 * IB * C::DB * 16 * kWave;   // [2][IB][64]
    float* xl = xm + 2 * IB * kWave;
    constexpr int NV = IB * C::DB * 16;
    for (int round = 0; round < 2; round++) {
        const int senders = round == 0 ? 2 : 1;     // waves [senders, 2*senders) send
        if (wave >= senders && wave < 2 * senders) {
            const int slot = wave - senders;
#pragma unroll
            for (int ib = 0; ib < IB; ib++) {
                xm[(slot * IB + ib) * kWave + lane] = m_run[ib];
                xl[(slot * IB + ib) * kWave + lane] = l_tot[ib];
#pragma unroll
                for (int db = 0; db < C::DB; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        xo[(slot * NV + (ib * C::DB + db) * 16 + r) * kWave + lane] = oacc[ib][db][r];
            }
        }
        __syncthreads();
        if (wave < senders) {
#pragma unroll
            for (int ib = 0; ib < IB; ib++) {
                const float mb = xm[(wave * IB + ib) * kWave + lane];
                const float lb = xl[(wave * IB + ib) * kWave + lane];
                const float M = fmaxf(m_run[ib], mb);
                const float wa = (m_run[ib] == -INFINITY) ? 0.f : fast_exp2(m_run[ib] - M);
                const float wb = (mb == -INFINITY) ? 0.f : fast_exp2(mb - M);
                l_tot[ib] = wa * l_tot[ib] + wb * lb;
                m_run[ib] = M;
#pragma unroll
                for (int db = 0; db < C::DB; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        oacc[ib][db][r] = wa * oacc[ib][db][r] +
                                          wb * xo[(wave * NV + (ib * C::DB + db) * 16 + r) * kWave + lane];
            }
        }
        __syncthreads();
    }

    if (wave != 0) return;
    const int n_chunks = gridDim.x;
#pragma unroll
    for (int ib = 0; ib < IB; ib++) {
        const int n = rb * 64 + ib * 32 + li;
        if (n >= N) continue;
        const size_t row = (size_t)(n / G) * a.Hq + kvh * G + n % G;
        const float inv = l_tot[ib] > 0.f ? 1.f / l_tot[ib] : 0.f;
        const float lse = l_tot[ib] > 0.f ? (m_run[ib] + __log2f(l_tot[ib])) * kLn2 : -INFINITY;
#pragma unroll
        for (int db = 0; db < C::DB; db++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++) {
                const int d0 = 32 * db + 8 * g4 + 4 * hi;
                const f32x4 v = f32x4{oacc[ib][db][4 * g4], oacc[ib][db][4 * g4 + 1],
                                      oacc[ib][db][4 * g4 + 2], oacc[ib][db][4 * g4 + 3]} * inv;
                if (n_chunks > 1) {
                    *(f32x4*)(a.ws_o + (row * n_chunks + c) * D + d0) = v;
                } else if (a.out_f32) {
                    *(f32x4*)((float*)a.o + row * D + d0) = v;
                } else {
                    *(u32x2*)((uint16_t*)a.o + row * D + d0) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                }
            }
        if (hi == 0) {
            if (n_chunks > 1) a.ws_lse[row * n_chunks + c] = lse;
            else if (a.lse) a.lse[row] = lse;
        }
    }
}

}  // namespace

size_t prefix_lds_bytes(int D) {
    return D == 64 ? 4 * PCfg<64>::WAVE_LDS : 4 * PCfg<128>::WAVE_LDS;
}

hipError_t launch_prefix(const PrefixArgs& a, hipStream_t stream) {
    const int N = a.R * (a.Hq / a.Hkv);
    const dim3 grid((a.prefix_len + a.chunk - 1) / a.chunk, a.Hkv, (N + 63) / 64);
    const size_t lds = prefix_lds_bytes(a.D);
    if (a.D == 64) {
        hipFuncSetAttribute((const void*)prefix_kernel<64>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        prefix_kernel<64><<<grid, 256, lds, stream>>>(a);
    } else {
        hipFuncSetAttribute((const void*)prefix_kernel<128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        prefix_kernel<128><<<grid, 256, lds, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace attn
