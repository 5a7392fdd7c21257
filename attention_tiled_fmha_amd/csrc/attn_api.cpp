// The C ABI of libattn.so (declared in include/attn.h): argument checks,
// split planning and kernel launches.  Every check runs on the host before
// anything is enqueued; on any error nothing is launched.  The library keeps
// no state between calls.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kPageSize = 16;
constexpr int kMaxSplit = 1024;    // longest chunk one workgroup takes
constexpr int kMinSplit = 64;      // 4 wavefronts x one 16-token page
constexpr int kGridYZ = 65535;

bool dim_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(int t) { return t == ATTN_BF16 || t == ATTN_F32; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }
// Tensors are read and written with 16-byte vector accesses; lse, tables,
// lengths and counters with 4-byte ones.  NULL passes (checked separately).
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int plan(int batch, int heads_kv, int max_kv_len, int num_cus, int requested, int* split,
         int* max_splits) {
    if (batch < 0 || heads_kv <= 0 || max_kv_len < 0) return ATTN_E_SHAPE;
    if (num_cus <= 0) num_cus = attn::device_cus();
    int s;
    if (requested > 0) {
        s = (requested + kMinSplit - 1) / kMinSplit * kMinSplit;
    } else {
        // The longest power-of-two chunk (64 .. 1024 tokens) that still
        // leaves at least num_cus (sequence, kv head, chunk) items at the
        // batch's worst case, batch * heads_kv * max_kv_len / s.  Measured
        // over batch 1..128 and contexts 1k..32k (D = 128): every item pays
        // a fixed start, so short chunks are slow, and this choice was the
        // fastest or within 4% of it on every shape.
        const double per_item = (double)batch * heads_kv * (double)max_kv_len / num_cus;
        s = kMinSplit;
        while (s < kMaxSplit && 2.0 * s <= per_item) s *= 2;
    }
    *split = s;
    *max_splits = max_kv_len > 0 ? (max_kv_len + s - 1) / s : 1;
    return ATTN_OK;
}

size_t decode_ws_bytes(int batch, int heads_q, int head_dim, int max_splits) {
    if (max_splits <= 1) return 0;
    const size_t rows = (size_t)batch * heads_q * max_splits;
    return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

int check_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

// The device scratch of attn_decode_paged_noalloc: the split partials of one
// call, in a fixed array that each GPU the library runs on holds until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the array is reached only through the per-device address
// that hipGetSymbolAddress returns (taken once per device, with that device
// current).
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Address of the current device's scratch array, or NULL on error.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

#if ATTN_CHECKED
// The checked build's device error word (bits kDevErrKvLen, kDevErrPage),
// one per GPU, reached like the scratch array through its per-device address.
static __device__ unsigned int dev_errors;
void* g_err_ptr[kMaxDevices] = {};
#endif

// Address of the current device's error word; NULL in the release build.
unsigned* device_error_word() {
#if ATTN_CHECKED
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_err_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(dev_errors)) != hipSuccess || !ptr) return nullptr;
        g_err_ptr[dev] = ptr;
    }
    return (unsigned*)g_err_ptr[dev];
#else
    return nullptr;
#endif
}

// Whole pages of page_bytes from p to the end of the device allocation that
// holds p: the bound the checked build holds page indices to (INT_MAX when
// the runtime knows no allocation at p).
int pool_pages(const void* p, size_t page_bytes) {
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (!p || page_bytes == 0 ||
        hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess || !base) {
        (void)hipGetLastError();
        return INT_MAX;
    }
    const size_t avail = (size_t)((const char*)base + size - (const char*)p);
    return (int)std::min<size_t>(avail / page_bytes, INT_MAX);
}

// The checked build's error word and pool bound for a call over the pools
// k_pages / v_pages of page_bytes per page (NULL and 0 in the release build,
// where the kernels compile the checks away).
void set_checks(unsigned** err, int* num_pages, const void* k_pages, const void* v_pages,
                size_t page_bytes) {
#if ATTN_CHECKED
    *err = device_error_word();
    *num_pages = std::min(pool_pages(k_pages, page_bytes), pool_pages(v_pages, page_bytes));
#else
    (void)k_pages;
    (void)v_pages;
    (void)page_bytes;
    *err = nullptr;
    *num_pages = 0;
#endif
}

// Flat GEMM planning, from sweeps of (rows, wavefronts, k slices) over the
// four decode projections of a Llama2-7B layer (n x k = 12288 x 4096,
// 4096 x 4096, 22016 x 4096, 4096 x 11008) at m = 1, 8, 16, 64:
//  - wavefronts per workgroup: 4 (more, smaller workgroups beat 8 on every
//    shape but one, by up to 15%);
//  - rows per workgroup: 16 for m <= 8, and for m <= 16 on weights of at
//    most 2^24 elements; 32 for m <= 32 when 64-row blocks alone would
//    number 1.25x the CUs (gate_up at m = 16: 47.5 us against 52.3); else
//    64 (four row blocks share every A fragment, so A is re-read from L2 a
//    quarter as often: 283 -> ~170 us per layer at m = 64);
//  - k slices across workgroups (fp32 partials plus a reduction launch of
//    ~4 us): with 16 rows, doubled while the row blocks alone leave CUs
//    idle, and 4 when the grid fills one to three rounds of resident
//    workgroups (the last round's tail shrinks: gate_up at m = 1 33 us
//    against 37); with 64 rows, none from 160 row blocks on (5/8 of the
//    CUs), else up to 4.  Every wavefront keeps at least one register
//    batch of 32-wide k steps (two with 64 rows).
constexpr int kFgMaxM = 64;
constexpr int kFgMaxK = 1 << 22;
constexpr int kFgLdsMaxK = 1 << 20;   // LDS-tiled kernel: 256 rows x k x 2 bytes stay in one descriptor
constexpr int kFgWaves = 4;
constexpr int kFgResident = 4;     // 4-wavefront workgroups resident per CU
constexpr int kFgChunk = 64;       // k per chunk of the LDS-tiled kernel

// The LDS-tiled kernel (m > 16): rows of W per workgroup and k slices.
// Measured on the Llama2-7B decode projections at m = 32, 48 and 64 (rows
// 64 / 128 / 256 against 1 .. 16 slices): 64 rows, or 128 on the widest
// weight (gate_up, n = 22016), with slices doubled until the grid holds at
// least two workgroups per CU, were the fastest or within 4% of it (m = 64:
// qkv 28.1 us with 4 slices, o 14.5 with 8, gate_up 45.9 with 128 rows and
// 4, down 26.4 with 8).  Every slice keeps at least 4 chunks.
void flat_gemm_lds_plan(int m, int n, int k, int num_cus, const attn_flat_gemm_opts* o,
                        int* rows, int* splits, int* chunks_per_split) {
    const int nchunks = std::max(1, (k + kFgChunk - 1) / kFgChunk);
    int tr = (o && o->rows_per_workgroup) ? o->rows_per_workgroup : 0;
    if (!tr) tr = n >= 16384 ? 128 : 64;
    const long tiles = (n + tr - 1) / tr;
    int s = (o && o->splits) ? o->splits : 0;
    if (!s) {
        s = 1;
        while (tiles * s < 2L * num_cus && s < nchunks / 4) s *= 2;
        s = std::max(1, std::min(s, std::max(1, nchunks / 4)));
    }
    s = std::max(1, std::min(s, nchunks));
    const int cps = (nchunks + s - 1) / s;
    *rows = tr;
    *chunks_per_split = cps;
    *splits = (nchunks + cps - 1) / cps;
    (void)m;
}

int flat_gemm_plan(int m, int n, int k, int num_cus, const attn_flat_gemm_opts* o, int* splits,
                   int* steps_per_split, int* row_blocks, int* waves, int* lds_rows = nullptr,
                   int* chunks_per_split = nullptr) {
    if (m < 0 || n < 0 || k < 0) return ATTN_E_SHAPE;
    if (o && (o->splits < 0 || o->rows_per_workgroup < 0 || o->waves_per_workgroup < 0 ||
              o->kernel < 0))
        return ATTN_E_SHAPE;
    if (m > kFgMaxM || k > kFgMaxK || k % 8) return ATTN_E_UNSUPPORTED;
    if (o && o->kernel > 2) return ATTN_E_UNSUPPORTED;
    const int fr = o ? o->rows_per_workgroup : 0;
    if (fr && fr != 16 && fr != 32 && fr != 64 && fr != 128 && fr != 256) return ATTN_E_UNSUPPORTED;
    if (o && o->waves_per_workgroup && o->waves_per_workgroup != 4 && o->waves_per_workgroup != 8)
        return ATTN_E_UNSUPPORTED;
    if (num_cus <= 0) num_cus = attn::device_cus();
    // which kernel: forced, else the LDS-tiled one for m > 16, and for
    // m >= 8 on weights above 2^24 elements (measured at m = 8 / 16: qkv 22.7
    // / 22.9 us against 25.6 / 27.3, gate_up 37.0 / 38.1 against 42.4 / 48.4,
    // down 22.9 / 23.2 against 22.6 / 26.6; on the 2^24-element o weight and
    // at m = 1 the register-streaming kernel stays ahead), unless the options
    // only fit the register-streaming one
    const int fk = o ? o->kernel : 0;
    const int fw = o ? o->waves_per_workgroup : 0;
    bool lds;
    if (fk == 2) {
        if (k > kFgLdsMaxK || (fr && fr < 64) || fw == 8) return ATTN_E_UNSUPPORTED;
        lds = true;
    } else if (fk == 1) {
        if (fr > 64) return ATTN_E_UNSUPPORTED;
        lds = false;
    } else {
        const bool shape = m > 16 || (m >= 8 && (long)n * k > (1L << 24));
        lds = fr > 64 || (shape && k <= kFgLdsMaxK && !(fr && fr < 64) && fw != 8);
    }
    if (lds) {
        int tr = 0, cps = 0;
        flat_gemm_lds_plan(m, n, k, num_cus, o, &tr, splits, &cps);
        *steps_per_split = 0;
        *row_blocks = tr / 16;
        *waves = 4;
        if (lds_rows) *lds_rows = tr;
        if (chunks_per_split) *chunks_per_split = cps;
        return ATTN_OK;
    }
    if (lds_rows) *lds_rows = 0;
    if (chunks_per_split) *chunks_per_split = 0;
    const int nw = (o && o->waves_per_workgroup) ? o->waves_per_workgroup : kFgWaves;
    int rb;
    if (o && o->rows_per_workgroup)
        rb = o->rows_per_workgroup / 16;
    else if (m <= 8 || (m <= 16 && (long)n * k <= (1L << 24)))
        rb = 1;
    else if (m <= 32 && (long)((n + 63) / 64) * 4 >= 5L * num_cus)
        rb = 2;
    else
        rb = 4;
    const long rblocks = (n + 16L * rb - 1) / (16L * rb);
    const int nsteps = (k + 31) / 32;
    const int U = attn::flat_gemm_batch_steps(std::max(m, 1), rb);
    int s = 1;
    if (o && o->splits > 0) {
        s = o->splits;
    } else if (rb == 1) {
        while (rblocks * s < num_cus && nsteps / (2L * s * nw) >= U) s *= 2;
        const long resident = (long)kFgResident * num_cus;
        if (s == 1 && rblocks > resident && rblocks < 3 * resident && nsteps / (4L * nw) >= U)
            s = 4;
    } else if (rb == 2) {
        while (s < 4 && rblocks * s < num_cus && nsteps / (2L * s * nw) >= 2 * U) s *= 2;
    } else if (rblocks * 8 < 5L * num_cus) {
        s = 4;
        while (s > 1 && nsteps / ((long)s * nw) < 2 * U) s /= 2;
    } else if (rblocks > num_cus && rblocks < 2L * num_cus && nsteps / (2L * nw) >= 2 * U) {
        // between one and two rounds of row blocks (e.g. gate_up at m = 64:
        // 344 on 256 CUs) two k slices even the rounds out: 72 against 79 us
        s = 2;
    }
    s = std::max(1, std::min(s, std::max(nsteps, 1)));
    const int sps = std::max(1, (nsteps + s - 1) / s);
    *steps_per_split = sps;
    *splits = std::max(1, (nsteps + sps - 1) / sps);
    *row_blocks = rb;
    *waves = nw;
    return ATTN_OK;
}

size_t flat_gemm_ws_bytes(int m, int n, int splits) {
    return splits > 1 ? align256((size_t)splits * m * n * sizeof(float)) : 0;
}

// Shared-prefix chunking: an item is (chunk, kv head, block of 32 query rows),
// one 4-wavefront workgroup each; aim for about one item per compute unit,
// in chunks of 64 .. 1024 tokens.  Measured on the 64-request, 4096-token
// prefix: one item per CU beats two or four, since each item pays a fixed
// start (queries, page table, first pages) and a cross-wave merge.
void prefix_plan(int batch, int heads_q, int heads_kv, int prefix_len, int* chunk, int* n_chunks) {
    const long rows = (long)batch * (heads_q / heads_kv);
    const long per_chunk = (long)heads_kv * ((rows + 31) / 32);
    const long want = std::max(1L, (1L * attn::device_cus() + per_chunk - 1) / per_chunk);
    long c = (prefix_len + want - 1) / want;
    c = std::min(1024L, std::max(64L, (c + 63) / 64 * 64));
    *chunk = (int)c;
    *n_chunks = (int)((prefix_len + c - 1) / c);
}

int decode_common(const void* q, const void* k_pages, const void* v_pages,
                  const int32_t* block_table, long bt_stride, const int32_t* kv_lens,
                  int fixed_len, void* o, float* lse, int batch, int heads_q, int heads_kv,
                  int head_dim, int page_size, int max_pages_per_seq, int max_kv_len, int dtype,
                  int o_dtype, float scale, void* workspace, size_t workspace_bytes,
                  void* stream, int requested_split, bool unified = false, float phi = 0.f,
                  int* fallback_count = nullptr, float k_scale = 1.f, float v_scale = 1.f,
                  bool use_scratch = false) {
    // dtype ATTN_FP8_E4M3: bf16 queries over an FP8 cache (matrix-core kernel only)
    const bool fp8 = dtype == ATTN_FP8_E4M3;
    if ((!fp8 && !dtype_ok(dtype)) || !dtype_ok(o_dtype)) return ATTN_E_UNSUPPORTED;
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || max_kv_len < 0 || max_pages_per_seq < 0)
        return ATTN_E_SHAPE;
    if (heads_q % heads_kv) return ATTN_E_SHAPE;
    if (!dim_ok(head_dim) || page_size != kPageSize) return ATTN_E_UNSUPPORTED;
    const int G = heads_q / heads_kv;
    if (G > 16) return ATTN_E_UNSUPPORTED;
    if ((long)max_pages_per_seq * page_size < max_kv_len) return ATTN_E_SHAPE;
    if (!scale_ok(scale) || !scale_ok(k_scale) || !scale_ok(v_scale)) return ATTN_E_ARG;
    if (batch == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !o || (!block_table && max_kv_len > 0))
        return ATTN_E_NULL;
    if (!al16(q) || !al16(k_pages) || !al16(v_pages) || !al16(o) || !al16(workspace) ||
        !al4(lse) || !al4(block_table) || !al4(kv_lens) || !al4(fallback_count))
        return ATTN_E_ARG;
    if (batch > kGridYZ || heads_kv > kGridYZ) return ATTN_E_UNSUPPORTED;
    int split = 0, max_splits = 0;
    const int rc = plan(batch, heads_kv, max_kv_len, 0, requested_split, &split, &max_splits);
    if (rc != ATTN_OK) return rc;
    const size_t need = decode_ws_bytes(batch, heads_q, head_dim, max_splits);
    if (use_scratch && need > 0) {   // attn_decode_paged_noalloc
        if (need > kScratchBytes) return ATTN_E_SCRATCH;
        if (!(workspace = device_scratch())) return ATTN_E_HIP;
        workspace_bytes = kScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;

    attn::DecodeArgs a{};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.kv_lens = kv_lens;
    a.fixed_len = fixed_len;
    a.max_len = max_kv_len;
    a.o = o;
    a.lse = lse;
    const size_t rows = (size_t)batch * heads_q * max_splits;
    a.ws_o = need ? (float*)workspace : nullptr;
    a.ws_lse = need ? (float*)((char*)workspace + align256(rows * head_dim * sizeof(float))) : nullptr;
    a.B = batch;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.D = head_dim;
    a.split_tokens = split;
    a.max_splits = max_splits;
    a.in_f32 = dtype == ATTN_F32;
    a.out_f32 = o_dtype == ATTN_F32;
    a.in_fp8 = fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.scale = scale;
    a.unified = unified;
    a.phi = phi;
    a.fallback_count = fallback_count;
    set_checks(&a.err, &a.num_pages, k_pages, v_pages,
               (size_t)heads_kv * kPageSize * head_dim * (fp8 ? 1 : dtype == ATTN_F32 ? 4 : 2));
    // bf16 and FP8 caches go to the matrix-core kernel; fp32 caches and
    // chunks longer than it takes go to the vector kernel (no unified-max
    // mode, no FP8, G in {1, 2, 4, 8})
    if (attn::decode_mfma_supported(a)) return check_hip(attn::launch_decode_mfma(a, (hipStream_t)stream));
    if (unified || fp8 || (G != 1 && G != 2 && G != 4 && G != 8)) return ATTN_E_UNSUPPORTED;
    return check_hip(attn::launch_decode(a, (hipStream_t)stream));
}

}  // namespace

namespace attn {

int device_cus() {
    constexpr int kFallback = 256, kMax = 64;
    static std::atomic<int> cached[kMax];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMax) return kFallback;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = kFallback;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace attn


extern "C" {

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_E_NULL: return "a required pointer is NULL";
        case ATTN_E_SHAPE: return "invalid or inconsistent sizes";
        case ATTN_E_UNSUPPORTED: return "unsupported configuration";
        case ATTN_E_WORKSPACE: return "workspace missing or too small";
        case ATTN_E_HIP: return "HIP launch error";
        case ATTN_E_ARG: return "argument value out of domain or misaligned pointer";
        case ATTN_E_SCRATCH:
            return "the call needs more scratch than the library's fixed device array holds";
        default: return "unknown status";
    }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                 int heads_q, int heads_kv, int seq_q, int seq_kv, int head_dim, int dtype,
                 int causal, float scale, void* stream) {
    if (!dtype_ok(dtype)) return ATTN_E_UNSUPPORTED;
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || seq_q < 0 || seq_kv < 0)
        return ATTN_E_SHAPE;
    if (heads_q % heads_kv) return ATTN_E_SHAPE;
    if (!dim_ok(head_dim)) return ATTN_E_UNSUPPORTED;
    if (!scale_ok(scale)) return ATTN_E_ARG;
    if (batch == 0 || seq_q == 0) return ATTN_OK;
    if (!q || !o || (seq_kv > 0 && (!k || !v))) return ATTN_E_NULL;
    if (!al16(q) || !al16(k) || !al16(v) || !al16(o) || !al4(lse)) return ATTN_E_ARG;
    if ((long)batch * heads_q * ((seq_q + 255) / 256) > 0x7fffffffL) return ATTN_E_UNSUPPORTED;
    hipError_t e;
    if (dtype == ATTN_F32)
        e = attn::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, (float*)o,
                                     lse, batch, heads_q, heads_kv, seq_q, seq_kv, head_dim,
                                     causal != 0, scale, (hipStream_t)stream);
    else
        e = attn::launch_prefill_bf16(q, k, v, o, lse, batch, heads_q, heads_kv, seq_q, seq_kv,
                                      head_dim, causal != 0, scale, (hipStream_t)stream);
    return check_hip(e);
}

int attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                       int batch, int heads_q, int heads_kv, int seq_q, int head_dim,
                       int page_size, int max_pages_per_seq, int dtype, int causal, float scale,
                       void* stream) {
    if (dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || seq_q < 0 || max_pages_per_seq < 0)
        return ATTN_E_SHAPE;
    if (heads_q % heads_kv) return ATTN_E_SHAPE;
    if (!dim_ok(head_dim) || page_size != kPageSize) return ATTN_E_UNSUPPORTED;
    if (!scale_ok(scale)) return ATTN_E_ARG;
    if (batch == 0 || seq_q == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !block_table || !kv_lens || !o) return ATTN_E_NULL;
    if (!al16(q) || !al16(k_pages) || !al16(v_pages) || !al16(o) || !al4(lse) ||
        !al4(block_table) || !al4(kv_lens))
        return ATTN_E_ARG;
    if ((long)batch * heads_q * ((seq_q + 255) / 256) > 0x7fffffffL) return ATTN_E_UNSUPPORTED;
    unsigned* err = nullptr;
    int num_pages = 0;
    set_checks(&err, &num_pages, k_pages, v_pages, (size_t)heads_kv * kPageSize * head_dim * 2);
    return check_hip(attn::launch_prefill_paged_bf16(q, k_pages, v_pages, block_table, kv_lens, o,
                                                     lse, batch, heads_q, heads_kv, seq_q,
                                                     head_dim, max_pages_per_seq, causal != 0,
                                                     scale, (hipStream_t)stream, err, num_pages));
}

int attn_decode_plan(int batch, int heads_kv, int max_kv_len, int num_cus, int requested_split,
                     int* split_tokens, int* max_splits) {
    if (!split_tokens || !max_splits) return ATTN_E_NULL;
    return plan(batch, heads_kv, max_kv_len, num_cus, requested_split, split_tokens, max_splits);
}

size_t attn_decode_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                   int max_kv_len, int split_tokens) {
    int split = 0, max_splits = 0;
    if (heads_q <= 0 || head_dim <= 0 ||
        plan(batch, heads_kv, max_kv_len, 0, split_tokens, &split, &max_splits) != ATTN_OK)
        return 0;
    return decode_ws_bytes(batch, heads_q, head_dim, max_splits);
}

int attn_decode_paged_ex(const void* q, const void* k_pages, const void* v_pages,
                         const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                         int batch, int heads_q, int heads_kv, int head_dim, int page_size,
                         int max_pages_per_seq, int max_kv_len, int dtype, int o_dtype,
                         float scale, void* workspace, size_t workspace_bytes, void* stream,
                         const attn_decode_opts* opts) {
    if (!dtype_ok(dtype)) return ATTN_E_UNSUPPORTED;   // FP8 caches: attn_decode_paged_fp8
    if (batch > 0 && !kv_lens) return ATTN_E_NULL;
    const int requested = opts ? opts->split_tokens : 0;
    if (requested < 0) return ATTN_E_ARG;
    const bool unified = opts && opts->use_unified_max;
    const float phi = opts ? opts->phi : 0.f;
    if (unified && !std::isfinite(phi)) return ATTN_E_ARG;
    return decode_common(q, k_pages, v_pages, block_table, max_pages_per_seq, kv_lens, 0, o,
                         lse, batch, heads_q, heads_kv, head_dim, page_size, max_pages_per_seq,
                         max_kv_len, dtype, o_dtype, scale, workspace, workspace_bytes, stream,
                         requested, unified, phi, opts ? opts->fallback_count : nullptr);
}

int attn_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* kv_lens, void* o,
                              float* lse, int batch, int heads_q, int heads_kv, int head_dim,
                              int page_size, int max_pages_per_seq, int max_kv_len, int dtype,
                              int o_dtype, float scale, void* stream) {
    if (!dtype_ok(dtype)) return ATTN_E_UNSUPPORTED;
    if (batch > 0 && !kv_lens) return ATTN_E_NULL;
    return decode_common(q, k_pages, v_pages, block_table, max_pages_per_seq, kv_lens, 0, o, lse,
                         batch, heads_q, heads_kv, head_dim, page_size, max_pages_per_seq,
                         max_kv_len, dtype, o_dtype, scale, nullptr, 0, stream, 0, false, 0.f,
                         nullptr, 1.f, 1.f, true);
}

int attn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages,
                          float k_scale, float v_scale, const int32_t* block_table,
                          const int32_t* kv_lens, void* o, float* lse, int batch, int heads_q,
                          int heads_kv, int head_dim, int page_size, int max_pages_per_seq,
                          int max_kv_len, int o_dtype, float scale, void* workspace,
                          size_t workspace_bytes, void* stream, const attn_decode_opts* opts) {
    if (batch > 0 && !kv_lens) return ATTN_E_NULL;
    const int requested = opts ? opts->split_tokens : 0;
    if (requested < 0) return ATTN_E_ARG;
    const bool unified = opts && opts->use_unified_max;
    const float phi = opts ? opts->phi : 0.f;
    if (unified && !std::isfinite(phi)) return ATTN_E_ARG;
    return decode_common(q, k_pages, v_pages, block_table, max_pages_per_seq, kv_lens, 0, o,
                         lse, batch, heads_q, heads_kv, head_dim, page_size, max_pages_per_seq,
                         max_kv_len, ATTN_FP8_E4M3, o_dtype, scale, workspace, workspace_bytes,
                         stream, requested, unified, phi, opts ? opts->fallback_count : nullptr,
                         k_scale, v_scale);
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* kv_lens, void* o, float* lse,
                      int batch, int heads_q, int heads_kv, int head_dim, int page_size,
                      int max_pages_per_seq, int max_kv_len, int dtype, int o_dtype,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return attn_decode_paged_ex(q, k_pages, v_pages, block_table, kv_lens, o, lse, batch,
                                heads_q, heads_kv, head_dim, page_size, max_pages_per_seq,
                                max_kv_len, dtype, o_dtype, scale, workspace, workspace_bytes,
                                stream, nullptr);
}

int attn_merge_states(void* o_a, float* lse_a, const void* o_b, const float* lse_b, int rows,
                      int head_dim, int o_dtype, void* stream) {
    if (!dtype_ok(o_dtype)) return ATTN_E_UNSUPPORTED;
    if (rows < 0) return ATTN_E_SHAPE;
    if (!dim_ok(head_dim)) return ATTN_E_UNSUPPORTED;
    if (rows == 0) return ATTN_OK;
    if (!o_a || !lse_a || !o_b || !lse_b) return ATTN_E_NULL;
    if (!al16(o_a) || !al16(o_b) || !al4(lse_a) || !al4(lse_b)) return ATTN_E_ARG;
    return check_hip(attn::launch_merge_states(o_a, lse_a, o_b, lse_b, rows, head_dim,
                                               o_dtype == ATTN_F32, (hipStream_t)stream));
}

size_t attn_shared_prefix_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                          int prefix_len, int dtype) {
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || heads_q % heads_kv || head_dim <= 0 ||
        prefix_len < 0)
        return 0;
    if ((dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3) && prefix_len > 0) {
        int chunk = 0, n_chunks = 0;
        prefix_plan(batch, heads_q, heads_kv, prefix_len, &chunk, &n_chunks);
        return decode_ws_bytes(batch, heads_q, head_dim, n_chunks);
    }
    int split = 0, max_splits = 0;
    if (plan(batch, heads_kv, prefix_len, 0, 0, &split, &max_splits) != ATTN_OK) return 0;
    return decode_ws_bytes(batch, heads_q, head_dim, max_splits);
}

static int shared_prefix_common(const void* q, const void* k_pages, const void* v_pages,
                         const int32_t* prefix_pages, int prefix_len, void* o, float* lse,
                         int batch, int heads_q, int heads_kv, int head_dim, int page_size,
                         int dtype, int o_dtype, float scale, void* workspace,
                         size_t workspace_bytes, void* stream, float k_scale, float v_scale) {
    const bool fp8 = dtype == ATTN_FP8_E4M3;
    if (prefix_len < 0) return ATTN_E_SHAPE;
    const int npages = (prefix_len + kPageSize - 1) / kPageSize;
    if (dtype == ATTN_F32 || prefix_len == 0) {
        // fp32 test mode (and the empty prefix): every request runs the paged
        // decode over the one shared table.
        return decode_common(q, k_pages, v_pages, prefix_pages, 0, nullptr, prefix_len, o, lse,
                             batch, heads_q, heads_kv, head_dim, page_size, npages, prefix_len,
                             dtype, o_dtype, scale, workspace, workspace_bytes, stream, 0, false,
                             0.f, nullptr, k_scale, v_scale);
    }
    if (!dtype_ok(o_dtype)) return ATTN_E_UNSUPPORTED;
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || heads_q % heads_kv) return ATTN_E_SHAPE;
    if (!dim_ok(head_dim) || page_size != kPageSize) return ATTN_E_UNSUPPORTED;
    if (!scale_ok(scale) || !scale_ok(k_scale) || !scale_ok(v_scale)) return ATTN_E_ARG;
    if (batch == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !prefix_pages || !o) return ATTN_E_NULL;
    if (!al16(q) || !al16(k_pages) || !al16(v_pages) || !al16(o) || !al16(workspace) ||
        !al4(lse) || !al4(prefix_pages))
        return ATTN_E_ARG;
    const long rows = (long)batch * (heads_q / heads_kv);
    if ((rows + 63) / 64 > kGridYZ || heads_kv > kGridYZ) return ATTN_E_UNSUPPORTED;
    int chunk = 0, n_chunks = 0;
    prefix_plan(batch, heads_q, heads_kv, prefix_len, &chunk, &n_chunks);
    const size_t need = decode_ws_bytes(batch, heads_q, head_dim, n_chunks);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
    const size_t nrow = (size_t)batch * heads_q * n_chunks;
    float* ws_o = need ? (float*)workspace : nullptr;
    float* ws_lse = need ? (float*)((char*)workspace + align256(nrow * head_dim * sizeof(float)))
                         : nullptr;

    attn::PrefixArgs a{};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.pages = prefix_pages;
    a.prefix_len = prefix_len;
    a.o = o;
    a.lse = lse;
    a.ws_o = ws_o;
    a.ws_lse = ws_lse;
    a.R = batch;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.D = head_dim;
    a.chunk = chunk;
    a.out_f32 = o_dtype == ATTN_F32;
    a.in_fp8 = fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.scale = scale;
    set_checks(&a.err, &a.num_pages, k_pages, v_pages,
               (size_t)heads_kv * kPageSize * head_dim * (fp8 ? 1 : 2));
    hipError_t e = attn::launch_prefix(a, (hipStream_t)stream);
    if (e != hipSuccess || n_chunks <= 1) return check_hip(e);

    attn::DecodeArgs c{};
    c.kv_lens = nullptr;
    c.fixed_len = prefix_len;
    c.max_len = prefix_len;
    c.o = o;
    c.lse = lse;
    c.ws_o = ws_o;
    c.ws_lse = ws_lse;
    c.B = batch;
    c.Hq = heads_q;
    c.Hkv = heads_kv;
    c.D = head_dim;
    c.split_tokens = chunk;
    c.max_splits = n_chunks;
    c.out_f32 = a.out_f32;
    return check_hip(attn::launch_decode_combine(c, (hipStream_t)stream));
}

int attn_decode_shared_prefix(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* prefix_pages, int prefix_len, void* o, float* lse,
                              int batch, int heads_q, int heads_kv, int head_dim, int page_size,
                              int dtype, int o_dtype, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return ATTN_E_UNSUPPORTED;   // FP8 caches: the _fp8 entry
    return shared_prefix_common(q, k_pages, v_pages, prefix_pages, prefix_len, o, lse, batch,
                                heads_q, heads_kv, head_dim, page_size, dtype, o_dtype, scale,
                                workspace, workspace_bytes, stream, 1.f, 1.f);
}

int attn_decode_shared_prefix_fp8(const void* q, const void* k_pages, const void* v_pages,
                                  float k_scale, float v_scale, const int32_t* prefix_pages,
                                  int prefix_len, void* o, float* lse, int batch, int heads_q,
                                  int heads_kv, int head_dim, int page_size, int o_dtype,
                                  float scale, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    return shared_prefix_common(q, k_pages, v_pages, prefix_pages, prefix_len, o, lse, batch,
                                heads_q, heads_kv, head_dim, page_size, ATTN_FP8_E4M3, o_dtype,
                                scale, workspace, workspace_bytes, stream, k_scale, v_scale);
}

int attn_flat_gemm_plan(int m, int n, int k, int num_cus, const attn_flat_gemm_opts* opts,
                        int* splits, int* rows_per_workgroup, int* kernel) {
    if (!splits || !rows_per_workgroup) return ATTN_E_NULL;
    int sps = 0, rb = 0, nw = 0, lr = 0, cps = 0;
    const int rc = flat_gemm_plan(m, n, k, num_cus, opts, splits, &sps, &rb, &nw, &lr, &cps);
    if (rc == ATTN_OK) {
        *rows_per_workgroup = 16 * rb;
        if (kernel) *kernel = lr > 0 ? 2 : 1;
    }
    return rc;
}

size_t attn_flat_gemm_workspace_bytes(int m, int n, int k, const attn_flat_gemm_opts* opts) {
    int s = 0, sps = 0, rb = 0, nw = 0;
    if (flat_gemm_plan(m, n, k, 0, opts, &s, &sps, &rb, &nw) != ATTN_OK) return 0;
    return flat_gemm_ws_bytes(m, n, s);
}

int attn_flat_gemm(const void* a, const void* w, void* c, int m, int n, int k, int dtype,
                   int c_dtype, void* workspace, size_t workspace_bytes, void* stream,
                   const attn_flat_gemm_opts* opts) {
    if (dtype != ATTN_BF16 || !dtype_ok(c_dtype)) return ATTN_E_UNSUPPORTED;
    int s = 0, sps = 0, rb = 0, nw = 0, lr = 0, cps = 0;
    const int rc = flat_gemm_plan(m, n, k, 0, opts, &s, &sps, &rb, &nw, &lr, &cps);
    if (rc != ATTN_OK) return rc;
    if (m == 0 || n == 0) return ATTN_OK;
    if (!c || (k > 0 && (!a || !w))) return ATTN_E_NULL;
    if (!al16(a) || !al16(w) || !al4(c) || !al16(workspace)) return ATTN_E_ARG;
    if ((long)((n + 15) / 16) * s > 0x7fffffffL) return ATTN_E_UNSUPPORTED;
    const size_t need = flat_gemm_ws_bytes(m, n, s);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
    attn::FlatGemmArgs p{};
    p.a = a;
    p.w = w;
    p.c = c;
    p.ws = (float*)workspace;
    p.m = m;
    p.n = n;
    p.k = k;
    p.splits = s;
    p.steps_per_split = sps;
    p.row_blocks = rb;
    p.waves = nw;
    p.lds_rows = lr;
    p.chunks_per_split = cps;
    p.out_f32 = c_dtype == ATTN_F32;
    return check_hip(attn::launch_flat_gemm(p, (hipStream_t)stream));
}

// Cascade in one call: the prefix stage (the dense prefix kernel, its chunks
// as the shared-prefix entry plans them) writes its chunk states to the first
// slots of every row of the decode workspace, the sequences' own chunks (the
// decode planner's split) follow them, and the decode's combine merges both,
// so neither the prefix chunk combine nor the state merge runs on its own.
static void cascade_plan(int batch, int heads_q, int heads_kv, int prefix_len, int max_suffix_len,
                         int* split, int* max_splits_s, int* prefix_chunk, int* prefix_slots) {
    plan(batch, heads_kv, max_suffix_len, 0, 0, split, max_splits_s);
    *prefix_chunk = 0;
    *prefix_slots = 0;
    if (prefix_len > 0) prefix_plan(batch, heads_q, heads_kv, prefix_len, prefix_chunk, prefix_slots);
}

size_t attn_cascade_workspace_bytes(int batch, int heads_q, int heads_kv, int head_dim,
                                    int prefix_len, int max_suffix_len, int dtype) {
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || heads_q % heads_kv || head_dim <= 0 ||
        prefix_len < 0 || max_suffix_len < 0 || (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3))
        return 0;
    int split = 0, ms = 0, pc = 0, ps = 0;
    cascade_plan(batch, heads_q, heads_kv, prefix_len, max_suffix_len, &split, &ms, &pc, &ps);
    return decode_ws_bytes(batch, heads_q, head_dim, ps + ms);
}

int attn_decode_cascade(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* prefix_pages, int prefix_len,
                        const int32_t* suffix_table, const int32_t* suffix_lens, void* o,
                        float* lse, int batch, int heads_q, int heads_kv, int head_dim,
                        int page_size, int max_pages_per_seq, int max_suffix_len, int dtype,
                        int o_dtype, float scale, float k_scale, float v_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
    const bool fp8 = dtype == ATTN_FP8_E4M3;
    if ((dtype != ATTN_BF16 && !fp8) || !dtype_ok(o_dtype)) return ATTN_E_UNSUPPORTED;
    if (batch < 0 || heads_q <= 0 || heads_kv <= 0 || prefix_len < 0 || max_suffix_len < 0 ||
        max_pages_per_seq < 0 || heads_q % heads_kv)
        return ATTN_E_SHAPE;
    if (!dim_ok(head_dim) || page_size != kPageSize) return ATTN_E_UNSUPPORTED;
    if (heads_q / heads_kv > 16) return ATTN_E_UNSUPPORTED;   // the decode kernel's group limit
    if ((long)max_pages_per_seq * page_size < max_suffix_len) return ATTN_E_SHAPE;
    if (!fp8) k_scale = v_scale = 1.f;
    if (!scale_ok(scale) || !scale_ok(k_scale) || !scale_ok(v_scale)) return ATTN_E_ARG;
    if (batch == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !o || (!prefix_pages && prefix_len > 0) ||
        (!suffix_table && max_suffix_len > 0))
        return ATTN_E_NULL;
    if (!al16(q) || !al16(k_pages) || !al16(v_pages) || !al16(o) || !al16(workspace) ||
        !al4(lse) || !al4(prefix_pages) || !al4(suffix_table) || !al4(suffix_lens))
        return ATTN_E_ARG;
    const long rows = (long)batch * (heads_q / heads_kv);
    if (batch > kGridYZ || heads_kv > kGridYZ || (rows + 63) / 64 > kGridYZ)
        return ATTN_E_UNSUPPORTED;
    int split = 0, ms = 0, pc = 0, ps = 0;
    cascade_plan(batch, heads_q, heads_kv, prefix_len, max_suffix_len, &split, &ms, &pc, &ps);
    const int slots = ps + ms;
    const size_t need = decode_ws_bytes(batch, heads_q, head_dim, slots);
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
    const size_t nrow = (size_t)batch * heads_q * slots;
    float* ws_o = need ? (float*)workspace : nullptr;
    float* ws_lse = need ? (float*)((char*)workspace + align256(nrow * head_dim * sizeof(float)))
                         : nullptr;

    if (ps > 0) {
        attn::PrefixArgs p{};
        p.q = q;
        p.k_pages = k_pages;
        p.v_pages = v_pages;
        p.pages = prefix_pages;
        p.prefix_len = prefix_len;
        p.ws_o = ws_o;
        p.ws_lse = ws_lse;
        p.R = batch;
        p.Hq = heads_q;
        p.Hkv = heads_kv;
        p.D = head_dim;
        p.chunk = pc;
        p.out_f32 = o_dtype == ATTN_F32;
        p.in_fp8 = fp8;
        p.k_scale = k_scale;
        p.v_scale = v_scale;
        p.scale = scale;
        p.ws_slots = slots;
        set_checks(&p.err, &p.num_pages, k_pages, v_pages,
                   (size_t)heads_kv * kPageSize * head_dim * (fp8 ? 1 : 2));
        const hipError_t e = attn::launch_prefix(p, (hipStream_t)stream);
        if (e != hipSuccess) return check_hip(e);
    }
    attn::DecodeArgs a{};
    a.q = q;
    a.k_pages = k_pages;
    a.v_pages = v_pages;
    a.block_table = suffix_table;
    a.bt_stride = max_pages_per_seq;
    a.kv_lens = suffix_lens;
    a.fixed_len = max_suffix_len;
    a.max_len = max_suffix_len;
    a.o = o;
    a.lse = lse;
    a.ws_o = ws_o;
    a.ws_lse = ws_lse;
    a.B = batch;
    a.Hq = heads_q;
    a.Hkv = heads_kv;
    a.D = head_dim;
    a.split_tokens = split;
    a.max_splits = slots;
    a.out_f32 = o_dtype == ATTN_F32;
    a.in_fp8 = fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.scale = scale;
    a.prefix_slots = ps;
    set_checks(&a.err, &a.num_pages, k_pages, v_pages,
               (size_t)heads_kv * kPageSize * head_dim * (fp8 ? 1 : 2));
    return check_hip(attn::launch_decode_mfma(a, (hipStream_t)stream));
}

int attn_checked_build(void) { return ATTN_CHECKED; }

int attn_device_errors(unsigned int* flags, int clear) {
#if ATTN_CHECKED
    if (!flags) return ATTN_E_NULL;
    unsigned* p = device_error_word();
    if (!p) return ATTN_E_HIP;
    unsigned v = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return ATTN_E_HIP;
    if (clear) {
        const unsigned z = 0;
        if (hipMemcpy(p, &z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return ATTN_E_HIP;
    }
    *flags = v;
    return ATTN_OK;
#else
    (void)flags;
    (void)clear;
    return ATTN_E_UNSUPPORTED;
#endif
}

int attn_device_pool_pages(const void* pages, size_t page_bytes, int* num_pages) {
    if (!num_pages) return ATTN_E_NULL;
    *num_pages = pool_pages(pages, page_bytes);
    return ATTN_OK;
}

int attn_probe_block_bytes(void) { return attn::hbm_probe_block_bytes(); }

int attn_probe_hbm_read(const void* buf, const int32_t* order, int n_blocks, uint32_t* sink,
                        void* stream) {
    if (n_blocks < 0) return ATTN_E_SHAPE;
    if (n_blocks == 0) return ATTN_OK;
    if (!buf || !sink) return ATTN_E_NULL;
    if (!al16(buf) || !al4(sink) || (order && !al4(order))) return ATTN_E_ARG;
    return check_hip(attn::launch_hbm_read(buf, order, n_blocks, sink, (hipStream_t)stream));
}

}  // extern "C"
