// kvx.hip -- host side of libkvx.so: argument validation, variant dispatch and
// one launch per call on the caller's stream.  The C ABI and its contract are
// declared and documented in include/kvx.h.
#include "kvx.h"
#include "kvx_kernels.hpp"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <vector>
#include <cstdlib>
#include <cstring>
#include <type_traits>

using namespace kvx;

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxRowBytes = 65536;

std::atomic<int> g_cus[kMaxDevices];

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("KVX_LOG");
        return e != nullptr && e[0] == '1';
    }();
    return on;
}

// Cap on workgroups per compute unit; beyond it the waves grid-stride over
// the chunks (a persistent grid).  0 (the default) means no cap: one wave per
// chunk.  Measured (same process, alternating) with the final chunk sizes: a
// cap of 2, 4 or 6 workgroups per CU makes the five-op step 8-21% slower
// (5895 GB/s uncapped vs 5425 / 5279 / 4633) and single ops up to 32%
// slower.  KVX_BLOCKS_PER_CU sets a cap, for experiments.
int blocks_per_cu() {
    static const int n = [] {
        const char* e = std::getenv("KVX_BLOCKS_PER_CU");
        if (e == nullptr) return 0;
        int v = std::atoi(e);
        return v < 0 ? 0 : v;
    }();
    return n;
}

kvx_status device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KVX_E_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        int n = g_cus[dev].load(std::memory_order_relaxed);
        if (n > 0) { *cus = n; return KVX_OK; }
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return KVX_E_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return KVX_OK;
}

int elem_bytes(int32_t dtype) {
    switch (dtype) {
        case KVX_F16: case KVX_BF16: return 2;
        case KVX_FP8: return 1;
        case KVX_F32: return 4;
        default: return 0;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b into *out, false on int64 overflow (a, b >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    return !__builtin_mul_overflow(a, b, out);
}

struct Geom {
    int32_t Q;
    int64_t R;       // row bytes
    int64_t Db;      // head_dim * element size
    int32_t H;
};

kvx_status check_layout(const kvx_layout* l, Geom* g) {
    if (l == nullptr) return KVX_E_NULL;
    const int eb = elem_bytes(l->dtype);
    if (eb == 0) return KVX_E_DTYPE;
    if (l->num_layers < 1 || l->num_kv < 1 || l->num_kv > 2 || l->kv_heads < 1 ||
        l->head_dim < 1)
        return KVX_E_SHAPE;
    int64_t Q = static_cast<int64_t>(l->num_layers) * l->num_kv;
    int64_t Db = static_cast<int64_t>(l->head_dim) * eb;
    int64_t R = 0;
    if (Q > (1 << 20)) return KVX_E_RANGE;
    if (!mul_ok(Db, l->kv_heads, &R) || R > kMaxRowBytes) return KVX_E_RANGE;
    if (R % 16 != 0) return KVX_E_ALIGN;
    g->Q = static_cast<int32_t>(Q);
    g->R = R;
    g->Db = Db;
    g->H = l->kv_heads;
    return KVX_OK;
}

// Bytes between consecutive pages of a plane (page_stride 0: page_size *
// slot_stride); -1 when that product overflows.
int64_t page_stride_of(const kvx_pool* p) {
    if (p->page_stride != 0) return p->page_stride;
    int64_t ps = 0;
    return mul_ok(p->page_size, p->slot_stride, &ps) ? ps : -1;
}

kvx_status check_pool(const kvx_pool* p, const Geom& g) {
    if (p == nullptr || p->planes == nullptr) return KVX_E_NULL;
    if (p->num_pages < 0 || p->page_size < 1 || p->slot_stride < g.R || p->page_stride < 0)
        return KVX_E_SHAPE;
    if (p->slot_stride % 16 != 0 || p->page_stride % 16 != 0) return KVX_E_ALIGN;
    // bytes of a page's rows; a nonzero page stride may not make pages overlap
    int64_t rows = 0;
    if (!mul_ok(p->page_size - 1, p->slot_stride, &rows) || rows > INT64_MAX - g.R)
        return KVX_E_RANGE;
    rows += g.R;
    if (p->page_stride != 0 && p->page_stride < rows) return KVX_E_SHAPE;
    if (p->page_stride % p->slot_stride != 0) return KVX_E_UNSUPPORTED;
    if (p->page_stride / p->slot_stride > INT32_MAX) return KVX_E_RANGE;
    const int64_t ps = page_stride_of(p);
    int64_t bytes = 0;                          // extent of one plane
    if (ps < 0 || (p->num_pages > 0 && (!mul_ok(p->num_pages - 1, ps, &bytes) ||
                                        bytes > INT64_MAX - rows)))
        return KVX_E_RANGE;
    if (p->num_pages > 0) bytes += rows;
    for (int32_t q = 0; q < g.Q; ++q) {
        if (p->planes[q] == nullptr) {
            if (bytes == 0) continue;            // an empty pool's planes may be NULL
            return KVX_E_NULL;
        }
        if (!aligned16(p->planes[q])) return KVX_E_ALIGN;
    }
    return KVX_OK;
}

// A source pool must hold at least one slot when there are tokens to move:
// rows that are not copied load the plane's first slot instead of a computed
// address.
kvx_status check_source_nonempty(const kvx_pool* p, const kvx_reqs* r) {
    if (r->total_tokens > 0 && (p->num_pages == 0 || p->page_size == 0)) return KVX_E_SHAPE;
    return KVX_OK;
}

kvx_status check_reqs(const kvx_reqs* r) {
    if (r == nullptr) return KVX_E_NULL;
    if (r->num_reqs < 0 || r->total_tokens < 0) return KVX_E_SHAPE;
    if (r->num_reqs == 0 && r->total_tokens != 0) return KVX_E_SHAPE;
    if (r->num_reqs > 0 && r->tok_off == nullptr) return KVX_E_NULL;
    if (r->total_tokens >= (int64_t(1) << 31)) return KVX_E_RANGE;
    return KVX_OK;
}

kvx_status check_table(const kvx_table* t, const kvx_reqs* r) {
    if (t == nullptr) return KVX_E_NULL;
    if (t->num_ids < 0) return KVX_E_SHAPE;
    if (r->num_reqs > 0 && t->pg_off == nullptr) return KVX_E_NULL;
    if (t->num_ids > 0 && t->page_ids == nullptr) return KVX_E_NULL;
    return KVX_OK;
}

void fill_pool_ref(PoolRef* ref, const kvx_pool* p, const kvx_table* t, int32_t q0, int32_t nq) {
    std::memset(ref, 0, sizeof(*ref));
    for (int32_t i = 0; i < nq; ++i) ref->plane[i] = static_cast<char*>(p->planes[q0 + i]);
    ref->stride = p->slot_stride;
    // the page step as an int32 row count beside page_size, with the page
    // shift derived in the kernel, keeps the pool descriptor at its former
    // size: one more 8-byte field per pool made the pool-to-pool kernel 1.5%
    // slower (measured, same process; the shift costs nothing)
    ref->page_rows = static_cast<int32_t>(page_stride_of(p) / p->slot_stride);
    ref->num_pages = p->num_pages;
    ref->pg_off = t->pg_off;
    ref->ids = t->page_ids;
    ref->num_ids = t->num_ids;
    ref->page_size = p->page_size;
}

// Chunk shape for a unit size: (VPL, U) for the wide copy, VPL = 0 for flat.
struct Shape {
    int vpl;
    uint32_t U;
};

// Rows per chunk of the wide copy for a row of vpl KiB.
template <int VPL>
constexpr int wide_rows() {
    return KVX_CHUNK_KIB / VPL > 0 ? KVX_CHUNK_KIB / VPL : 1;
}

Shape shape_for(int64_t unit_bytes) {
    if (unit_bytes % 1024 == 0) {
        switch (unit_bytes / 1024) {
            case 1: return {1, static_cast<uint32_t>(wide_rows<1>())};
            case 2: return {2, static_cast<uint32_t>(wide_rows<2>())};
            case 4: return {4, static_cast<uint32_t>(wide_rows<4>())};
            case 8: return {8, static_cast<uint32_t>(wide_rows<8>())};
            case 16: return {16, static_cast<uint32_t>(wide_rows<16>())};
            default: break;
        }
    }
    int64_t u = kChunkBytes / unit_bytes;
    if (u < 1) u = 1;
    if (u > kWave) u = kWave;
    return {0, static_cast<uint32_t>(u)};
}

// Waves of these kernels (<= 64 VGPRs) that one compute unit holds at once.
constexpr int64_t kResidentWavesPerCu = 32;

// Rows per chunk for the wide copies (paged rows and permute token rows of
// 1..16 KiB).  A launch that fits in one round of resident waves at 8 KiB
// chunks keeps them (every wave runs at once, with the most loads in flight
// per lane); a larger one moves the fewest rows that make wave_bytes per wave
// (one row when the row is that large), so that the waves still running when
// the launch drains are short.  Measured on MI355X (same process,
// alternating): 8 KiB chunks win below one round (gather of 128 144 KiB
// tokens: 3610 vs 3373 GB/s; extract of 58.7 MB: 6253 vs 5877), one row per
// wave wins above it for the permutes (extract of 470 MB: 5380 -> 5924-6045;
// rebuild 5414 -> 6192; just over one round, extract of 75 MB: 5364 -> 6444)
// and 2 KiB per wave for the paged ops: 2 KiB rows one per wave (scatter of
// 302 MB 5214 -> 5378; fragmented gather of 7 GB 5127 -> 5314; two per wave
// loses 2-4%), 1 KiB rows two per wave (gather-scatter of 537 MB 3866 ->
// 5192 against one per wave, gather 5092 -> 5791, scatter 5326 -> 5607; four
// per wave 5185 / 5459 / 5416).
bool above_one_round(int64_t bytes, int cus) {
    return bytes > static_cast<int64_t>(cus) * kResidentWavesPerCu * kChunkBytes;
}

uint32_t wide_rows_for(const Shape& sh, int64_t rows, int64_t row_bytes, int cus,
                       int64_t wave_bytes) {
    if (sh.vpl <= 0 || sh.U == 1) return sh.U;
    if (!above_one_round(rows * row_bytes, cus)) return sh.U;
    return row_bytes >= wave_bytes ? 1u : static_cast<uint32_t>(wave_bytes / row_bytes);
}

// A paged launch with fewer chunks than the GPU has compute units leaves
// units idle: its chunks shrink -- U halves for the flat and row-loop copies,
// the wide copy steps to its next smaller instance (1 KiB rows 8 -> 2 -> 1,
// 2 KiB rows 4 -> 1, 4 KiB rows 2 -> 1) -- until there is at least one chunk
// per compute unit or one row per chunk.  Measured (same process, graph-
// timed, microseconds before -> after; gather-scatter / gather / scatter):
// 512-byte rows of 56 planes, 16 tokens 5.03 -> 4.43 / 4.73 -> 4.14 / 4.12
// -> 3.37, 32 tokens 5.04 -> 4.55 / 4.77 -> 4.31 / 4.26 -> 3.51, 64 tokens
// 5.07 -> 4.80 / 4.80 -> 4.54 / 4.32 -> 3.87; 1 KiB rows, 16 tokens 3.48 ->
// 3.15 / 3.28 -> 2.99 / 3.21 -> 2.90, 32 tokens 3.57 -> 3.63 / 3.44 -> 3.23 /
// 3.30 -> 3.01; 2 KiB rows of 72 planes, 4 tokens 3.29 -> 2.88 / 3.13 ->
// 2.72 / 3.08 -> 2.69; 1152-byte rows of 27 planes, 8 tokens 3.18 -> 2.78 /
// 2.97 -> 2.57 / 2.72 -> 2.41; launches with a chunk per unit unchanged.
// Asking for two or four chunks per unit gained less.
uint32_t rows_for_cus(const Shape& sh, int64_t tokens, int32_t nq, int cus) {
    uint32_t u = sh.U;
    auto chunks = [&](uint32_t k) {
        return (static_cast<uint64_t>(tokens) + k - 1) / k * static_cast<uint64_t>(nq);
    };
    while (u > 1 && chunks(u) < static_cast<uint64_t>(cus)) {
        if (sh.vpl == 1) u = u == 8 ? 2u : 1u;
        else if (sh.vpl > 1) u = 1u;
        else u /= 2;
    }
    return u;
}

// Small permute launches take smaller chunks too: token rows one row per
// chunk while the launch would have fewer than two 4-wave workgroups per
// compute unit, head rows (flat copy) U halved while it has fewer chunks than
// compute units.  Measured (same process, graph-timed, microseconds before
// -> after; extract / rebuild; 56 planes unless stated): 1 KiB token rows,
// seq 32 5.62 -> 2.50 / 3.53 -> 2.43, seq 128 7.82 -> 4.24 / 4.20 -> 4.09,
// seq 256 10.20 -> 7.31 / 6.73 -> 7.07; 2 KiB rows of 72 planes, seq 64
// 6.05 -> 4.76 / 5.16 -> 4.53; 4 KiB rows of 32 planes, seq 64 4.95 -> 4.63
// / 4.37 -> 4.24; 256-byte head rows (two heads), seq 16 4.35 -> 3.80 / 4.35
// -> 3.79, seq 64 4.45 -> 4.19 / 4.43 -> 4.22.  Larger launches keep their
// chunks (4 KiB rows at seq 128, one row per chunk: 6.79 -> 7.46 / 5.99 ->
// 6.86; head rows held to eight chunks per unit lose up to 50%).
uint32_t permute_rows_for_cus(const Shape& sh, bool token_rows, int64_t units, int32_t nq,
                              int cus) {
    auto chunks = [&](uint32_t k) {
        return (static_cast<uint64_t>(units) + k - 1) / k * static_cast<uint64_t>(nq);
    };
    uint32_t u = sh.U;
    if (token_rows) return u > 1 && chunks(u) < 8ull * static_cast<uint64_t>(cus) ? 1u : u;
    while (u > 1 && chunks(u) < static_cast<uint64_t>(cus)) u /= 2;
    return u;
}

// Paged rows of 4, 8 or 16 KiB in a launch above one round move as 2 KiB
// pieces (k_paged_sub): log2 of the pieces per row, 0 for whole rows (and when
// the launch's piece count would not fit the chunk index).  Measured (same process,
// alternating, whole rows against pieces, 256 MiB each way, page 1): 4 KiB
// rows gather-scatter 4830 -> 5205 GB/s, gather 6547 -> 6654, scatter 5175 ->
// 5321; 8 KiB rows 4984 -> 5152, 6498 -> 6710, 5269 -> 5463; 16 KiB rows
// 5009 -> 5081, 6427 -> 6717, 5223 -> 5414.
uint32_t sub_shift_for(const Shape& sh, int64_t tokens, int32_t nq, int64_t row_bytes,
                       int cus) {
    if (sh.vpl < 4 || !above_one_round(tokens * nq * row_bytes, cus)) return 0;
    const uint32_t shift = sh.vpl == 4 ? 1u : (sh.vpl == 8 ? 2u : 3u);
    const uint64_t chunks = (static_cast<uint64_t>(tokens) << shift) * static_cast<uint64_t>(nq);
    return chunks < (uint64_t(1) << 31) ? shift : 0u;
}

// A gather's staging holds each request's planes one after another, n_r
// rows per plane.  When requests are short -- on average at most 64 KiB of
// rows per plane -- token-major chunk order (the planes of a token block on
// adjacent waves) writes each request's block in longer runs than
// plane-major order does.  Measured (same process, alternating; 49152 or
// 65536 tokens in 64 .. 24576 equal requests, page-1 pools of 65536 slots):
// 2 KiB rows, 32 tokens per request 5164 -> 5672 GB/s, 16 tokens 4991 ->
// 5580, one token 4905 -> 5696, while 96 tokens lose (5679 -> 5261) and one
// request of 49152 tokens loses 16%; 512-byte rows, 128 tokens 5431 -> 5789,
// 256 tokens 5566 -> 5448; 1152-byte rows, 32 tokens 5207 -> 5463.  The
// scatter, which reads the staging, gains at most 5% and loses up to 5%
// (512-byte rows), so it keeps plane-major order.
constexpr int64_t kShortStageRunBytes = 64 << 10;

bool short_stage_runs(const kvx_reqs* reqs, int64_t row_bytes) {
    return reqs->num_reqs > 1 &&
           reqs->total_tokens * row_bytes <= kShortStageRunBytes * reqs->num_reqs;
}

// Bytes a wave of a large paged launch moves (see wide_rows_for); permutes
// move one row per wave.
constexpr int64_t kPagedWaveBytes = 2048;

// XCD-aware renumbering pays when a launch spans more memory than the
// translation caches reach: then each XCD, working on ~1/8 of the planes,
// touches ~1/8 of the translations.  Below that it costs a few percent.
// Measured (same process, alternating; a large pool's rate also moves by up
// to 8% between allocations, so only same-process pairs are compared):
// the 2048-token request in 4.5 GiB pools, gather-scatter 5015 GB/s without
// vs 4880 with; the same request spread over 36 GiB pools 4632 without vs
// 4798 with, and 131072 tokens there 5374 vs 5743; the fragmented gather
// from an 18 GiB pool 5082 vs 5322; a head-sliced copy over 13.5 GiB 5330
// vs 5114; permutes of 0.1-0.9 GB 3-9% faster without.  Pool-to-pool
// launches (two pools) renumber above a 16 GiB span: with two 9 GiB pools
// the page-1 gather-scatter is 4% faster without (5236 vs 5030).
constexpr double kRemapSpanBytes = 16.0 * (1ull << 30);
// Launches with one pool side (gather, scatter: the other side is staging)
// renumber from a pool of 8 GiB: with a 9 GiB pool gather runs 5409 -> 5651
// GB/s and scatter 5327 -> 5464 with it, and 4.5 GiB pools gain nothing.
constexpr double kRemapOnePoolBytes = 8.0 * (1ull << 30);

uint32_t remap_for(double span_bytes, double threshold = kRemapSpanBytes) {
    if (KVX_XCD_REMAP == 0) return 0;
    if (KVX_XCD_REMAP == 1) return 1;
    return span_bytes > threshold ? 1u : 0u;
}

// Lowest and highest base address among planes q0 .. q0 + nq - 1 of a pool.
void plane_range(const kvx_pool* p, int32_t q0, int32_t nq, uintptr_t* lo, uintptr_t* hi) {
    *lo = *hi = reinterpret_cast<uintptr_t>(p->planes[q0]);
    for (int32_t q = q0 + 1; q < q0 + nq; ++q) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p->planes[q]);
        *lo = b < *lo ? b : *lo;
        *hi = b > *hi ? b : *hi;
    }
}

// Bytes of planes q0 .. q0 + nq - 1 of a pool that a launch may touch: nq
// planes of num_slots * slot_stride bytes, or less when the planes overlap
// (a token-major pool, whose planes interleave slot by slot), where the
// planes' own address range is the bound.
double pool_span(const kvx_pool* p, int32_t q0, int32_t nq) {
    const double plane = static_cast<double>(p->num_pages) *
                         static_cast<double>(page_stride_of(p));
    uintptr_t lo = 0, hi = 0;
    plane_range(p, q0, nq, &lo, &hi);
    const double range = static_cast<double>(hi - lo) + plane;
    return range < plane * nq ? range : plane * nq;
}

// True when every plane base of the launch lies within one slot stride of
// the others: the rows of one slot in all planes then form one run of about
// slot_stride bytes (a token-major pool).  The paged kernels take
// token-major chunk order when the pool they write is such a pool, or, in a
// pool-to-pool copy, when either pool is.  Measured on the 2048-token,
// 144 KiB/token request with token-major 4.5 GiB pools (same process, the
// two orders alternating launch by launch, GB/s plane-major -> token-major,
// both with XCD renumbering): gather-scatter 4777 -> 5422, scatter 5135 ->
// 5393, gather from such a pool into staging 6554 -> 6495 (so a gather
// keeps plane-major order); token-major source into a layer-major pool
// 4869 -> 5151, and the reverse 4850 -> 5300.  With both sides
// layer-major, plane-major order is the faster one (five-op step 5902 vs
// 5706).
bool slot_interleaved(const kvx_pool* p, int32_t q0, int32_t nq) {
    if (p == nullptr || nq < 2) return false;
    uintptr_t lo = 0, hi = 0;
    plane_range(p, q0, nq, &lo, &hi);
    return static_cast<int64_t>(hi - lo) < p->slot_stride;
}

// DRAM-page order (dram_order in the kernels): two rows of one plane share
// an HBM DRAM page when they are a multiple of kDramSegBytes apart inside one
// aligned block of 4 * kDramSegBytes, and HBM serves them together when one
// XCD requests them together.  Measured with the library's kernels on the
// 2048-token, 144 KiB/token request at its density (2048 of 32768 slots per
// page-1 pool, 2 KiB rows; same process, designs alternating): rows in pairs
// 32 or 64 KiB apart on consecutive tokens 5904 / 5872 GB/s gather-scatter
// against 5125 for random slots; pairs 8-24, 48 or 128 KiB apart 5040-5069;
// the partner 2-8 tokens later (another XCD) 5013-5156.  So in a launch that
// moves one 2 KiB row, or two 1 KiB rows, per wave above one round of
// resident waves, a pool side whose pages hold runs of at least two segments
// of a plane has its rows one segment apart put on the two waves of one
// workgroup (1 KiB rows: in one wave).  Measured (same process, this build
// against the same sources built with KVX_DRAM_ORDER=0; 4.5 GiB pools, 8
// disjoint requests rotated, GB/s gather-scatter / gather / scatter): 2 KiB
// rows, 2048 tokens, pages of 32 rows 5578 -> 6071 / 6157 -> 6467 / 5916 ->
// 6268, of 64 rows 5878 -> 6127 / 6206 -> 6404 / 6080 -> 6332, of 128 rows
// 5949 -> 6024 / 6320 -> 6345 / 6086 -> 6267; 1 KiB rows, 2048 tokens, pages
// of 64 rows 5108 -> 5277 / 5599 -> 5833 / 5199 -> 5365; pages of 16 rows
// (not grouped) unchanged.  Launches within one round (8 KiB chunks of 2-8
// rows) lose 1.5-5% with the rows of a chunk grouped (2 KiB rows, 128
// tokens, pages of 32: 3948 -> 3820 gather-scatter): the whole launch is in
// flight at once, and a chunk's rows one segment apart all fall on one
// channel set where consecutive rows would have spread over several; they
// keep the natural order.
constexpr int64_t kDramSegBytes = 32 << 10;
#ifndef KVX_DRAM_ORDER
#define KVX_DRAM_ORDER 1           // 0: natural token order always (a build-time switch)
#endif

// True when a pool side can take the paired order for rows of R bytes: R a
// power of two of at most half a segment, rows contiguous within a page
// (slot stride R, pages not interleaved with other planes), page_size a
// multiple of two segments' tokens, and every plane base of the launch
// aligned to two segments (so that each pair lies in one DRAM block).
bool dram_pairs(const kvx_pool* p, int32_t q0, int32_t nq, int64_t R) {
    if (p == nullptr || R <= 0 || (R & (R - 1)) != 0 || R > kDramSegBytes / 2) return false;
    if (p->slot_stride != R || page_stride_of(p) != static_cast<int64_t>(p->page_size) * R)
        return false;
    const int64_t K = 2 * (kDramSegBytes / R);
    if (p->page_size % K != 0) return false;
    for (int32_t q = q0; q < q0 + nq; ++q)
        if (reinterpret_cast<uintptr_t>(p->planes[q]) % static_cast<uintptr_t>(2 * kDramSegBytes) != 0)
            return false;
    return true;
}

// The order word's DRAM-page bits (pairs: m = 2) for a plane-major paged
// launch of the wide copy with U rows of R bytes per chunk, or of 4-16 KiB
// rows in 2 KiB pieces (`pieces`; k_paged_sub pairs the same piece of two
// rows); `stage`: the staging buffer of a gather or scatter, else nullptr.
// 0 when the launch keeps the natural order.  Pieces measured (same process,
// against KVX_DRAM_ORDER=0; 2048 tokens, 16384-slot pools, 8 disjoint
// requests rotated; gather-scatter / gather / scatter GB/s): 4 KiB rows,
// pages of 16 rows 5514 -> 6084 / 6092 -> 6371 / 5879 -> 6259, of 32 rows
// 5824 -> 6074 / 6184 -> 6351 / 6057 -> 6263; 8 KiB rows, pages of 8 rows
// 5433 -> 6037 / 6063 -> 6376 / 5841 -> 6231, of 16 rows 5699 -> 6069 /
// 6131 -> 6320 / 6014 -> 6276; 16 KiB rows, pages of 4 rows 5330 -> 5982 /
// 6021 -> 6351 / 5790 -> 6233; page-1 pools (staging only) within 2.5%.
// The contiguous staging of a gather or scatter pairs the same way when its
// base is aligned to two segments (each request's plane blocks then pair
// too when their offsets are): measured (same process, against the order
// without it; GB/s gather / scatter): the 2048-token, 144 KiB/token request
// 6031 -> 6096 / 5544 -> 5584, 4096 tokens 5842 -> 5929 / 5386 -> 5488, 8
// requests of 1024 tokens 5747 -> 5849 / 5421 -> 5548, 4 ragged requests
// 5742 -> 5794 / 5386 -> 5438; 1 KiB rows, 4096 tokens 5777 -> 5759 / 5282
// -> 5475.
// Pools whose blocks hold the K and V pages of a layer together ([survey]
// 7.4's block length: a [num_blocks][2][B][H][D] tensor per layer, or one
// [num_blocks][L][2][B][H][D] tensor; planes 2l and 2l + 1 one page apart):
// with pages of 32 or 64 KiB, K row t and V row t of a block share a DRAM
// page, so planes pair instead of tokens (order bit 1, paged_chunk: the two
// planes of a token on the two waves of one workgroup).  Measured (same
// process, against KVX_DRAM_ORDER=0; one [blocks][36][2][B][8][128] bf16
// tensor per pool, 8 disjoint requests rotated; gather-scatter / scatter
// GB/s): pages of 16 rows (32 KiB), 2048 tokens 5048 -> 5958 / 5520 ->
// 5802, 4096 tokens 5157 -> 6146 / 5564 -> 5964, 8192 tokens 5185 -> 6197 /
// 5599 -> 5837; pages of 32 rows 5483 -> 5993 / 5856 -> 5847; 1 KiB rows,
// pages of 32 rows 5006 -> 5757 / 5308 -> 5254; pages of 8 rows (16 KiB, not
// paired) unchanged.  True when every plane pair of the launch (the launch
// starts at an even plane) is one page apart and each block's pair is
// aligned to its own length.
bool dram_plane_pairs(const kvx_pool* p, int32_t q0, int32_t nq, int64_t R) {
    if (p == nullptr || nq < 2 || (q0 & 1) != 0 || p->slot_stride != R) return false;
    const int64_t run = static_cast<int64_t>(p->page_size) * R;
    if (run % kDramSegBytes != 0 || 2 * run > 4 * kDramSegBytes) return false;
    if (page_stride_of(p) % (2 * run) != 0) return false;
    for (int32_t q = q0; q + 1 < q0 + nq; q += 2) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p->planes[q]);
        const uintptr_t b = reinterpret_cast<uintptr_t>(p->planes[q + 1]);
        if (b < a || b - a != static_cast<uintptr_t>(run) ||
            a % static_cast<uintptr_t>(2 * run) != 0)
            return false;
    }
    return true;
}

// Token-major pools (a slot's rows of all planes one run of Q R bytes): rows
// of planes g = 32 KiB / R apart lie one segment apart in that run, so in
// token-major order with one row per chunk the planes pair like tokens do in
// a block pool (order bit 2, paged_chunk).  Measured (same process, against
// the plain token-major order; 4.5 GiB pools of 2 KiB rows, 72 planes, 8
// disjoint requests rotated; gather-scatter GB/s): both pools token-major,
// 2048 tokens 5607 -> 5779, 8192 tokens 5777 -> 5961, page 16 6002 -> 6087;
// token-major into layer-major 5213 -> 5322, the reverse 5311 -> 5378;
// scatter into a token-major pool 5653 -> 5683.  Bits for a token-major
// launch that writes a pool (a gather of short requests, the other
// token-major launch, was not measured with it); 0 to keep the plane order.
#ifndef KVX_DRAM_TMAJOR
#define KVX_DRAM_TMAJOR 1
#endif
uint32_t tmajor_pair_bits(const kvx_pool* src, const kvx_pool* dst, int32_t q0, int32_t nq,
                          int64_t R, uint32_t U) {
    if (KVX_DRAM_ORDER == 0 || KVX_DRAM_TMAJOR == 0 || U != 1 || dst == nullptr) return 0;
    if (R <= 0 || (R & (R - 1)) != 0 || R > kDramSegBytes / 2) return 0;
    const int64_t g = kDramSegBytes / R;
    if (2 * g > nq) return 0;
    auto tm = [&](const kvx_pool* p) {
        return p != nullptr && p->slot_stride >= 2 * g * R && slot_interleaved(p, q0, nq);
    };
    if (!tm(src) && !tm(dst)) return 0;
    return 4u | (static_cast<uint32_t>(__builtin_ctzll(static_cast<uint64_t>(g))) << 8);
}

#ifndef KVX_DRAM_STAGE
#define KVX_DRAM_STAGE 1
#endif
uint32_t dram_order_bits(const kvx_pool* src, const kvx_pool* dst, int32_t q0, int32_t nq,
                         int64_t R, const Shape& sh, bool above_round, const void* stage,
                         bool pieces) {
    if (KVX_DRAM_ORDER == 0 || !above_round) return 0;
    if (!pieces && (sh.vpl <= 0 || sh.U * R > kPagedWaveBytes)) return 0;
    // plane pairs for gather-scatter and scatter; a gather keeps its staging
    // rows paired instead (its waves would otherwise write two planes'
    // staging blocks, n_r rows apart, at once: 8192 tokens of K/V blocks
    // gathered 5994 -> 5750 GB/s with plane pairs, while 2048 and 4096
    // tokens gained 2-3%)
    if (!pieces && dst != nullptr &&
        (dram_plane_pairs(src, q0, nq, R) || dram_plane_pairs(dst, q0, nq, R)))
        return 2u;
    const bool stage_ok = KVX_DRAM_STAGE != 0 && stage != nullptr && (R & (R - 1)) == 0 &&
                          R <= kDramSegBytes / 2 &&
                          reinterpret_cast<uintptr_t>(stage) % (2 * kDramSegBytes) == 0;
    if (!dram_pairs(src, q0, nq, R) && !dram_pairs(dst, q0, nq, R) && !stage_ok) return 0;
    const uint32_t gs = static_cast<uint32_t>(__builtin_ctzll(static_cast<uint64_t>(kDramSegBytes / R)));
    return (gs << 8) | (1u << 16);
}

// Paged ops only: rows of 512 B .. 16 KiB that are not a power-of-two number
// of KiB use the row-loop copy (vpl = -KMAX, U rows per chunk, U <= the
// instance's maximum).
Shape paged_shape_for(int64_t R) {
    Shape sh = shape_for(R);
    if (sh.vpl != 0 || R <= 512 || R > 16384) return sh;
    int kmax = 1;
    while (static_cast<int64_t>(kmax) * 1024 < R) kmax *= 2;
    int64_t umax = KVX_CHUNK_KIB / kmax > 0 ? KVX_CHUNK_KIB / kmax : 1;
    int64_t u = kChunkBytes / R;
    if (u < 1) u = 1;
    if (u > umax) u = umax;
    return {-kmax, static_cast<uint32_t>(u)};
}

// Fill the shape-dependent fields of Common; false if the chunk count overflows.
bool set_chunks(Common* c, const Shape& sh, uint32_t units_per_plane, int32_t nq) {
    c->U = sh.U;
    c->units_per_plane = units_per_plane;
    c->chunks_per_plane = (units_per_plane + sh.U - 1) / sh.U;
    uint64_t n = static_cast<uint64_t>(c->chunks_per_plane) * static_cast<uint64_t>(nq);
    if (n >= (uint64_t(1) << 31)) return false;
    c->nchunks = static_cast<uint32_t>(n);
    c->V = static_cast<uint32_t>(c->R / 16);
    c->v_magic = c->V == 1 ? 0u
                           : static_cast<uint32_t>(((uint64_t(1) << 32) + c->V - 1) / c->V);
    return true;
}

// Workgroups of wpb waves for one wave per chunk (or the cap).
uint32_t grid_for(uint32_t nchunks, int cus, int wpb) {
    uint64_t need = (static_cast<uint64_t>(nchunks) + wpb - 1) / wpb;
    uint64_t g = need;
    int bpc = blocks_per_cu();
    if (bpc > 0) {
        uint64_t cap = static_cast<uint64_t>(cus) * bpc;
        if (g > cap) g = cap;
    }
    if (g >= kXcds) g = (g + kXcds - 1) / kXcds * kXcds;   // XCD renumbering needs G % 8 == 0
    if (g < 1) g = 1;
    return static_cast<uint32_t>(g);
}

// lds: dynamic LDS bytes per workgroup.  The kernels use no LDS; a nonzero
// value only limits how many workgroups a compute unit holds at once.
template <class Args>
kvx_status launch(const void* fn, uint32_t grid, int wpb, Args& a, hipStream_t stream,
                  size_t lds = 0) {
    void* params[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kWave * wpb), params, lds, stream);
    return e == hipSuccess ? KVX_OK : KVX_E_HIP;
}

// Scatters above one round of resident waves run at 10 workgroups (20 waves)
// per compute unit instead of 16: 16 KiB of LDS per workgroup, out of 160 KiB
// per CU.  Fewer scattered row writes in flight at once go faster: measured
// on the 2048-token, 144 KiB/token request (same process, alternating,
// 4.5 GiB pools), scatter 5378 GB/s at full occupancy, 5439 / 5612 / 5570 at
// 13 / 10 / 8 workgroups per CU, and the five-op step 5585 -> 5644.  The
// other paged ops lose with the same cap (gather-scatter 5061 -> 4699 at 10,
// gather 5739 -> 5556).  Re-measured with the DRAM-page orders (scatter GB/s
// at pads 0 / 12 / 16 / 20 KiB, same process): 2 KiB rows page 1, 2048
// tokens 5390 / 5432 / 5669 / 5736, 8192 tokens 5480 / 5503 / 5584 / 5619;
// pages of 32 rows 6074 / 6210 / 6251 / 6055, of 16 rows 5096 / 5290 / 5825
// / 5795; 1 KiB rows 5523 / 5599 / 5506 / 5291; 4 KiB rows in 16-row pages
// 6152 / 6266 / 6289 / 6104: 16 KiB stays.
#ifndef KVX_SCATTER_LDS_PAD
#define KVX_SCATTER_LDS_PAD 16384
#endif
constexpr size_t kScatterLdsPad = KVX_SCATTER_LDS_PAD;

template <class Src, class Dst, bool MANY, bool NTS>
const void* paged_kernel_of(int vpl, uint32_t U) {
    const bool one = U == 1;
    switch (vpl) {
        case 1: return one      ? reinterpret_cast<const void*>(&k_paged<Src, Dst, 1, 1, MANY, NTS>)
                       : U == 2 ? reinterpret_cast<const void*>(&k_paged<Src, Dst, 1, 2, MANY, NTS>)
                                : reinterpret_cast<const void*>(&k_paged<Src, Dst, 1, wide_rows<1>(), MANY, NTS>);
        case 2: return one ? reinterpret_cast<const void*>(&k_paged<Src, Dst, 2, 1, MANY, NTS>)
                           : reinterpret_cast<const void*>(&k_paged<Src, Dst, 2, wide_rows<2>(), MANY, NTS>);
        case 4: return one ? reinterpret_cast<const void*>(&k_paged<Src, Dst, 4, 1, MANY, NTS>)
                           : reinterpret_cast<const void*>(&k_paged<Src, Dst, 4, wide_rows<4>(), MANY, NTS>);
        case 8: return reinterpret_cast<const void*>(&k_paged<Src, Dst, 8, wide_rows<8>(), MANY, NTS>);
        case 16: return reinterpret_cast<const void*>(&k_paged<Src, Dst, 16, wide_rows<16>(), MANY, NTS>);
        case -1: return reinterpret_cast<const void*>(&k_paged<Src, Dst, -1, wide_rows<1>(), MANY, NTS>);
        case -2: return reinterpret_cast<const void*>(&k_paged<Src, Dst, -2, wide_rows<2>(), MANY, NTS>);
        case -4: return reinterpret_cast<const void*>(&k_paged<Src, Dst, -4, wide_rows<4>(), MANY, NTS>);
        case -8: return reinterpret_cast<const void*>(&k_paged<Src, Dst, -8, wide_rows<8>(), MANY, NTS>);
        case -16: return reinterpret_cast<const void*>(&k_paged<Src, Dst, -16, wide_rows<16>(), MANY, NTS>);
        default: return reinterpret_cast<const void*>(&k_paged<Src, Dst, 0, 0, MANY, NTS>);
    }
}

// Batches of more than 64 requests take the kernels whose lookup first finds
// the chunk's 64-request window (a guessed one, else by a 64-way search);
// smaller ones the kernels whose one window holds the whole batch.  Stores
// are nontemporal unless the output is a staging the caller asked to be
// written with ordinary stores (`cached`; pool rows are never).
template <class Src, class Dst>
const void* paged_kernel(int vpl, uint32_t U, int32_t num_reqs, bool cached) {
    if constexpr (std::is_same<Dst, StageRef>::value) {
        if (cached)
            return num_reqs > kWave ? paged_kernel_of<Src, Dst, true, false>(vpl, U)
                                    : paged_kernel_of<Src, Dst, false, false>(vpl, U);
    }
    return num_reqs > kWave ? paged_kernel_of<Src, Dst, true, true>(vpl, U)
                            : paged_kernel_of<Src, Dst, false, true>(vpl, U);
}

template <class Src, class Dst>
const void* paged_sub_kernel(int32_t num_reqs, bool cached) {
    if constexpr (std::is_same<Dst, StageRef>::value) {
        if (cached)
            return num_reqs > kWave
                       ? reinterpret_cast<const void*>(&k_paged_sub<Src, Dst, true, false>)
                       : reinterpret_cast<const void*>(&k_paged_sub<Src, Dst, false, false>);
    }
    return num_reqs > kWave ? reinterpret_cast<const void*>(&k_paged_sub<Src, Dst, true, true>)
                            : reinterpret_cast<const void*>(&k_paged_sub<Src, Dst, false, true>);
}

template <int KT>
const void* heads_hnd_kernel(bool many) {
    return many ? reinterpret_cast<const void*>(&k_heads_hnd<KT, true>)
                : reinterpret_cast<const void*>(&k_heads_hnd<KT, false>);
}

// Token-row permute kernel for rows of vpl KiB; nullptr for the head-row
// (flat) kernel.
template <bool REBUILD, bool NTS>
const void* permute_rows_kernel(int vpl, uint32_t U) {
    const bool one = U == 1;
    switch (vpl) {
        case 1: return one ? reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 1, 1, NTS>)
                           : reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 1, wide_rows<1>(), NTS>);
        case 2: return one ? reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 2, 1, NTS>)
                           : reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 2, wide_rows<2>(), NTS>);
        case 4: return one ? reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 4, 1, NTS>)
                           : reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 4, wide_rows<4>(), NTS>);
        case 8: return reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 8, wide_rows<8>(), NTS>);
        case 16: return reinterpret_cast<const void*>(&k_permute_rows<REBUILD, 16, wide_rows<16>(), NTS>);
        default: return nullptr;
    }
}

const char* op_name(int op) {
    static const char* names[] = {"gather", "scatter", "gather_scatter"};
    return names[op];
}

// Shared body of the three paged calls.  Exactly one of (src pool, staging
// source) and one of (dst pool, staging destination) is set.
template <class Src, class Dst>
kvx_status run_paged(int op, const Geom& g, const kvx_reqs* reqs,
                     const kvx_pool* src, const kvx_table* st, void* src_stage,
                     const kvx_pool* dst, const kvx_table* dt, void* dst_stage,
                     unsigned long long* skipped, hipStream_t stream,
                     uint32_t out_cached = 0) {
    if (reqs->total_tokens == 0) return KVX_OK;           // nothing to move
    int cus = 0;
    kvx_status s = device_cus(&cus);
    if (s != KVX_OK) return s;
    const Shape sh0 = paged_shape_for(g.R);
    for (int32_t q0 = 0; q0 < g.Q; q0 += kTab) {
        const int32_t nq = g.Q - q0 < kTab ? g.Q - q0 : kTab;
        Shape sh = sh0;
        sh.U = wide_rows_for(sh0, reqs->total_tokens * nq, g.R, cus, kPagedWaveBytes);
        sh.U = rows_for_cus(sh, reqs->total_tokens, nq, cus);
        const uint32_t sub = sub_shift_for(sh0, reqs->total_tokens, nq, g.R, cus);
        if (sub > 0) sh = {2, 1};                 // one 2 KiB piece per chunk
        PagedArgs<Src, Dst> a;
        std::memset(&a, 0, sizeof(a));
        a.c.tok_off = reqs->tok_off;
        a.c.skipped = skipped;
        a.c.T = reqs->total_tokens;
        a.c.num_reqs = reqs->num_reqs;
        a.c.req_rate = static_cast<double>(reqs->num_reqs) /
                       static_cast<double>(reqs->total_tokens);
        a.c.q0 = q0;
        a.c.Q = g.Q;
        a.c.R = static_cast<int32_t>(g.R);
        a.c.sub_shift = sub;
        if (!set_chunks(&a.c, sh, static_cast<uint32_t>(reqs->total_tokens << sub), nq))
            return KVX_E_RANGE;
        if constexpr (std::is_same<Src, PoolRef>::value) fill_pool_ref(&a.src, src, st, q0, nq);
        else a.src.base = static_cast<char*>(src_stage);
        if constexpr (std::is_same<Dst, PoolRef>::value) fill_pool_ref(&a.dst, dst, dt, q0, nq);
        else a.dst.base = static_cast<char*>(dst_stage);
        a.c.remap = src != nullptr && dst != nullptr
                        ? remap_for(pool_span(src, q0, nq) + pool_span(dst, q0, nq))
                        : remap_for(pool_span(src != nullptr ? src : dst, q0, nq),
                                    kRemapOnePoolBytes);
        const bool tmajor = sub == 0 && (slot_interleaved(dst, q0, nq) ||
                                         (dst != nullptr && slot_interleaved(src, q0, nq)) ||
                                         (std::is_same<Dst, StageRef>::value &&
                                          short_stage_runs(reqs, g.R)));
        // token-major order renumbers at any size, so that each XCD takes whole
        // tokens' runs rather than every eighth row of each: measured on the
        // token-major 4.5 GiB pools (alternating launch by launch), gather-
        // scatter 5310 -> 5419 GB/s, scatter 5368 -> 5415
        if (tmajor && KVX_XCD_REMAP != 0) a.c.remap = 1;
        a.c.order = tmajor ? 1u | tmajor_pair_bits(src, dst, q0, nq, g.R, sh.U)
                           : dram_order_bits(src, dst, q0, nq, g.R, sh,
                                             above_one_round(reqs->total_tokens * nq * g.R, cus),
                                             src_stage != nullptr ? src_stage : dst_stage,
                                             sub > 0);
        const uint32_t grid = grid_for(a.c.nchunks, cus, kPagedWaves);
        const size_t lds = std::is_same<Src, StageRef>::value &&
                                   above_one_round(reqs->total_tokens * nq * g.R, cus)
                               ? kScatterLdsPad : 0;
        if (log_enabled())
            std::fprintf(stderr,
                         "kvx: %s Q=%d planes[%d,%d) R=%lld T=%lld reqs=%d copy=%s U=%u "
                         "pieces/row=%u chunks=%u grid=%u remap=%u order=%s dram_group=%u "
                         "lds_pad=%d stores=%s\n",
                         op_name(op), g.Q, q0, q0 + nq, static_cast<long long>(g.R),
                         static_cast<long long>(reqs->total_tokens), reqs->num_reqs,
                         sh.vpl > 0 ? "wide" : (sh.vpl < 0 ? "row-loop" : "flat"), sh.U,
                         1u << sub, a.c.nchunks, grid, a.c.remap,
                         tmajor ? ((a.c.order & 4u) != 0 ? "token-major-pairs" : "token-major")
                                : ((a.c.order & 2u) != 0 ? "plane-pairs" : "plane-major"),
                         (a.c.order >> 16) != 0 ? 1u << (a.c.order >> 16) : 0u,
                         static_cast<int>(lds),
                         std::is_same<Dst, StageRef>::value && out_cached != 0 ? "cached"
                                                                                : "nontemporal");
        const void* fn = sub > 0 ? paged_sub_kernel<Src, Dst>(a.c.num_reqs, out_cached != 0)
                                 : paged_kernel<Src, Dst>(sh.vpl, sh.U, a.c.num_reqs,
                                                          out_cached != 0);
        s = launch(fn, grid, kPagedWaves, a, stream, lds);
        if (s != KVX_OK) return s;
    }
    return KVX_OK;
}

// Permutes (perm_dram_order): with one token row per wave above one round,
// the four waves of a workgroup take the token rows that share DRAM pages on
// both sides: rows 32 KiB apart in the flat buffer, a head's rows 32 KiB
// apart in the HF tensors.  Measured (same process, against the natural
// order; three buffers rotated; extract / rebuild GB/s): 4 heads of 256 B
// (1 KiB token rows, the Qwen2.5-7B shape), seq 8192 6084-6118 -> 6376-6392
// / 5904-5908 -> 6303-6338, seq 4096 5951 -> 6219 / 5976 -> 6275; but 8
// heads (2 KiB rows) seq 2048 6359 -> 6027 / 6343 -> 6381, seq 8192 6207 ->
// 5989 / 6370 -> 6327, and 16 heads 6082 -> 5795 / 6058 -> 5968.  Pairing
// only the flat side's rows, or only the HF side's, moved none of these by
// more than 3% either way.  So only 4-head 1 KiB token rows take it.
#ifndef KVX_DRAM_PERMUTE
#define KVX_DRAM_PERMUTE 1
#endif
uint32_t permute_order_bits(const Geom& g, uint32_t U) {
    if (KVX_DRAM_ORDER == 0 || KVX_DRAM_PERMUTE == 0 || U != 1) return 0;
    if (g.H != 4 || g.R != 1024) return 0;
    const uint32_t ds = static_cast<uint32_t>(__builtin_ctzll(static_cast<uint64_t>(kDramSegBytes / g.R)));
    const uint32_t hs = static_cast<uint32_t>(__builtin_ctz(static_cast<uint32_t>(g.H)));
    return 8u | (ds << 8) | (hs << 16);
}

template <bool REBUILD>
kvx_status run_permute(const Geom& g, void* const* hf, int64_t s_cap, int64_t seq, void* flat,
                       uint32_t out_cached, hipStream_t stream) {
    if (seq == 0) return KVX_OK;
    int cus = 0;
    kvx_status s = device_cus(&cus);
    if (s != KVX_OK) return s;
    // Whole token rows (H * Db bytes) when they are 1..16 KiB powers of two;
    // otherwise head rows of Db bytes with the flat copy.
    const Shape tok = shape_for(g.R);
    const bool rows = tok.vpl > 0;
    const Shape sh0 = rows ? tok : shape_for(g.Db);
    const uint32_t units = static_cast<uint32_t>(rows ? seq : seq * g.H);
    for (int32_t q0 = 0; q0 < g.Q; q0 += kTab) {
        const int32_t nq = g.Q - q0 < kTab ? g.Q - q0 : kTab;
        Shape sh = sh0;
        if (rows) sh.U = wide_rows_for(sh0, seq * nq, g.R, cus, 0);
        sh.U = permute_rows_for_cus(sh, rows, units, nq, cus);
        PermuteArgs a;
        std::memset(&a, 0, sizeof(a));
        a.c.T = seq;
        a.c.q0 = q0;
        a.c.Q = g.Q;
        a.c.R = static_cast<int32_t>(g.Db);
        if (!set_chunks(&a.c, sh, units, nq)) return KVX_E_RANGE;
        for (int32_t i = 0; i < nq; ++i) a.hf[i] = static_cast<char*>(hf[q0 + i]);
        a.flat = static_cast<char*>(flat);
        a.s_cap = s_cap;
        a.H = g.H;
        a.c.remap = remap_for(static_cast<double>(nq) * g.H * s_cap * g.Db +
                              static_cast<double>(nq) * seq * g.R);
        if (rows) a.c.order = permute_order_bits(g, sh.U);
        const uint32_t grid = grid_for(a.c.nchunks, cus, kPermuteWaves);
        if (log_enabled())
            std::fprintf(stderr,
                         "kvx: %s Q=%d planes[%d,%d) H=%d Db=%lld seq=%lld s_cap=%lld unit=%s "
                         "U=%u chunks=%u grid=%u order=%s stores=%s\n",
                         REBUILD ? "rebuild" : "extract", g.Q, q0, q0 + nq, g.H,
                         static_cast<long long>(g.Db), static_cast<long long>(seq),
                         static_cast<long long>(s_cap), rows ? "token-row" : "head-row", sh.U,
                         a.c.nchunks, grid, (a.c.order & 8u) != 0 ? "dram-pages" : "natural",
                         out_cached != 0 ? "cached" : "nontemporal");
        // nontemporal stores unless the caller reads the output back soon
        const void* fn =
            out_cached == 0
                ? (rows ? permute_rows_kernel<REBUILD, true>(sh.vpl, sh.U)
                        : reinterpret_cast<const void*>(&k_permute<REBUILD, true>))
                : (rows ? permute_rows_kernel<REBUILD, false>(sh.vpl, sh.U)
                        : reinterpret_cast<const void*>(&k_permute<REBUILD, false>));
        s = launch(fn, grid, kPermuteWaves, a, stream);
        if (s != KVX_OK) return s;
    }
    return KVX_OK;
}

kvx_status check_heads(const kvx_heads* h, const kvx_pool* p, const Geom& g) {
    if (h == nullptr) return KVX_E_NULL;
    if (h->block_layout != KVX_NHD && h->block_layout != KVX_HND) return KVX_E_SHAPE;
    if (h->kv_heads < 1 || h->head0 < 0 || static_cast<int64_t>(h->head0) + g.H > h->kv_heads)
        return KVX_E_SHAPE;
    if (p->slot_stride < static_cast<int64_t>(h->kv_heads) * g.Db) return KVX_E_SHAPE;
    int64_t page_bytes = 0, pool_bytes = 0;
    if (!mul_ok(p->slot_stride, p->page_size, &page_bytes) ||
        !mul_ok(page_bytes, p->num_pages, &pool_bytes))
        return KVX_E_RANGE;
    // head-sliced copies address whole pages of one plane's rows only
    if (p->page_stride != 0 && p->page_stride != page_bytes) return KVX_E_UNSUPPORTED;
    return KVX_OK;
}

// Both sides NHD: a head slice of a token row is nh * Db contiguous bytes at
// offset head0 * Db of the row, so the slice copy is the row copy with plane
// bases moved by head0 * Db (each pool's slot stride unchanged).
kvx_status run_heads_as_rows(const Geom& g, const kvx_reqs* reqs, const kvx_pool* src,
                             const kvx_table* st, const kvx_heads* sh, const kvx_pool* dst,
                             const kvx_table* dt, const kvx_heads* dh,
                             unsigned long long* skipped, hipStream_t stream) {
    std::vector<void*> sp(static_cast<size_t>(g.Q)), dp(static_cast<size_t>(g.Q));
    for (int32_t q = 0; q < g.Q; ++q) {
        sp[q] = static_cast<char*>(src->planes[q]) + static_cast<int64_t>(sh->head0) * g.Db;
        dp[q] = static_cast<char*>(dst->planes[q]) + static_cast<int64_t>(dh->head0) * g.Db;
    }
    kvx_pool s2 = *src, d2 = *dst;
    s2.planes = sp.data();
    d2.planes = dp.data();
    return run_paged<PoolRef, PoolRef>(2, g, reqs, &s2, st, nullptr, &d2, dt, nullptr, skipped,
                                       stream);
}

kvx_status run_heads(const Geom& g, const kvx_reqs* reqs, const kvx_pool* src,
                     const kvx_table* st, const kvx_heads* sh, const kvx_pool* dst,
                     const kvx_table* dt, const kvx_heads* dh, unsigned long long* skipped,
                     hipStream_t stream) {
    if (reqs->total_tokens == 0) return KVX_OK;
    if (sh->block_layout == KVX_NHD && dh->block_layout == KVX_NHD)
        return run_heads_as_rows(g, reqs, src, st, sh, dst, dt, dh, skipped, stream);
    int cus = 0;
    kvx_status s = device_cus(&cus);
    if (s != KVX_OK) return s;
    // HND on both sides with one page size B <= 64: chunks of B tokens x nhc
    // heads (k_heads_hnd) when B * Db / 16 is 64, 128, 256 or 512 vectors and
    // Db / 16 is a power of two; otherwise chunks of Ut tokens x nhc heads of
    // Db-byte units with the flat copy (k_heads).
    const int64_t vd = g.Db / 16;
    const int64_t bv = static_cast<int64_t>(src->page_size) * vd;
    int kt = 0;
    if (sh->block_layout == KVX_HND && dh->block_layout == KVX_HND &&
        src->page_size == dst->page_size && src->page_size <= kWave &&
        (vd & (vd - 1)) == 0 && (bv == 64 || bv == 128 || bv == 256 || bv == 512))
        kt = static_cast<int>(bv / 64);
    int64_t units = kChunkBytes / g.Db;
    if (units < 1) units = 1;
    if (units > kWave) units = kWave;
    int32_t nhc0 = static_cast<int32_t>(g.H < units ? g.H : units);
    int32_t Ut0 = static_cast<int32_t>(units / nhc0);
    if (kt > 0) {
        Ut0 = src->page_size;                              // one page of tokens
        const int64_t per_head = Ut0 * g.Db;
        int64_t hc = kChunkBytes / per_head;
        if (hc < 1) hc = 1;
        nhc0 = static_cast<int32_t>(g.H < hc ? g.H : hc);
    }
    for (int32_t q0 = 0; q0 < g.Q; q0 += kTab) {
        const int32_t nq = g.Q - q0 < kTab ? g.Q - q0 : kTab;
        // a launch with fewer chunks than compute units takes smaller ones, as
        // the row kernels do: fewer tokens per chunk (flat copy), else fewer
        // heads (the page-run kernel's chunk is one page of tokens).  Measured
        // (same process, graph-timed, heads 4..7 of 8 into 0..3 of 4, 72
        // planes, one request): 8 tokens, HND -> NHD 5.34 -> 4.80 us, HND ->
        // HND 3.42 -> 3.31; 16 tokens at page 1, 5.40 -> 5.13; from 32 tokens
        // unchanged
        auto chunks_of = [&](int32_t ut, int32_t nc) {
            return (static_cast<uint64_t>(reqs->total_tokens) + ut - 1) / ut *
                   static_cast<uint64_t>((g.H + nc - 1) / nc) * static_cast<uint64_t>(nq);
        };
        int32_t Ut = Ut0, nhc = nhc0;
        while (chunks_of(Ut, nhc) < static_cast<uint64_t>(cus)) {
            if (kt == 0 && Ut > 1) Ut /= 2;
            else if (nhc > 1) nhc = (nhc + 1) / 2;
            else break;
        }
        const int32_t hblocks = (g.H + nhc - 1) / nhc;
        const uint64_t tblocks = (static_cast<uint64_t>(reqs->total_tokens) + Ut - 1) / Ut;
        HeadArgs a;
        std::memset(&a, 0, sizeof(a));
        a.c.tok_off = reqs->tok_off;
        a.c.skipped = skipped;
        a.c.T = reqs->total_tokens;
        a.c.num_reqs = reqs->num_reqs;
        a.c.req_rate = static_cast<double>(reqs->num_reqs) /
                       static_cast<double>(reqs->total_tokens);
        a.c.q0 = q0;
        a.c.Q = g.Q;
        a.c.R = static_cast<int32_t>(g.Db);
        a.c.U = static_cast<uint32_t>(Ut * nhc);
        const uint64_t cpp = tblocks * static_cast<uint64_t>(hblocks);
        const uint64_t n = cpp * static_cast<uint64_t>(nq);
        if (n >= (uint64_t(1) << 31)) return KVX_E_RANGE;
        a.c.chunks_per_plane = static_cast<uint32_t>(cpp);
        a.c.nchunks = static_cast<uint32_t>(n);
        a.c.V = static_cast<uint32_t>(g.Db / 16);
        a.c.v_magic = a.c.V == 1 ? 0u
                                 : static_cast<uint32_t>(((uint64_t(1) << 32) + a.c.V - 1) / a.c.V);
        fill_pool_ref(&a.src, src, st, q0, nq);
        fill_pool_ref(&a.dst, dst, dt, q0, nq);
        a.hs = HeadSide{sh->kv_heads, sh->head0, sh->block_layout == KVX_HND ? 1 : 0};
        a.hd = HeadSide{dh->kv_heads, dh->head0, dh->block_layout == KVX_HND ? 1 : 0};
        a.nh = g.H;
        a.nhc = nhc;
        a.Ut = Ut;
        a.hblocks = hblocks;
        a.head_major = (a.hs.hnd && a.hd.hnd) ? 1 : 0;
        a.c.remap = remap_for(pool_span(src, q0, nq) + pool_span(dst, q0, nq));
        if (kt > 0) a.c.U = static_cast<uint32_t>(Ut);
        const uint32_t grid = grid_for(a.c.nchunks, cus, kPagedWaves);
        if (log_enabled())
            std::fprintf(stderr,
                         "kvx: gather_scatter_heads Q=%d planes[%d,%d) nh=%d Db=%lld T=%lld "
                         "src(H=%d h0=%d %s) dst(H=%d h0=%d %s) Ut=%d nhc=%d kt=%d chunks=%u "
                         "grid=%u\n",
                         g.Q, q0, q0 + nq, g.H, static_cast<long long>(g.Db),
                         static_cast<long long>(reqs->total_tokens), a.hs.H, a.hs.h0,
                         a.hs.hnd ? "HND" : "NHD", a.hd.H, a.hd.h0, a.hd.hnd ? "HND" : "NHD",
                         Ut, nhc, kt, a.c.nchunks, grid);
        const bool many = a.c.num_reqs > kWave;
        const void* fn = many ? reinterpret_cast<const void*>(&k_heads<true>)
                              : reinterpret_cast<const void*>(&k_heads<false>);
        switch (kt) {
            case 1: fn = heads_hnd_kernel<1>(many); break;
            case 2: fn = heads_hnd_kernel<2>(many); break;
            case 4: fn = heads_hnd_kernel<4>(many); break;
            case 8: fn = heads_hnd_kernel<8>(many); break;
            default: break;
        }
        s = launch(fn, grid, kPagedWaves, a, stream);
        if (s != KVX_OK) return s;
    }
    return KVX_OK;
}

// Output flags a call accepts (KVX_E_UNSUPPORTED for any other bit).
kvx_status check_out_flags(uint32_t flags) {
    return (flags & ~static_cast<uint32_t>(KVX_OUT_CACHED)) == 0 ? KVX_OK : KVX_E_UNSUPPORTED;
}

kvx_status check_staging(const void* p, int64_t bytes, const Geom& g, const kvx_reqs* r) {
    int64_t need = 0;
    if (!mul_ok(r->total_tokens, static_cast<int64_t>(g.Q) * g.R, &need)) return KVX_E_RANGE;
    if (need > 0 && p == nullptr) return KVX_E_NULL;
    if (!aligned16(p)) return KVX_E_ALIGN;
    if (bytes < need) return KVX_E_SHAPE;
    return KVX_OK;
}

kvx_status check_hf(const Geom& g, const void* const* hf, int64_t s_cap, int64_t seq) {
    if (hf == nullptr) return KVX_E_NULL;
    if (s_cap < 0 || seq < 0 || seq > s_cap) return KVX_E_SHAPE;
    if (g.Db % 16 != 0) return KVX_E_ALIGN;
    // every product checked before it is used: head rows of the call below
    // 2^31, and one plane's [H, s_cap, D] bytes within int64
    int64_t units = 0, cap_rows = 0, plane_bytes = 0;
    if (!mul_ok(seq, g.H, &units) || units >= (int64_t(1) << 31)) return KVX_E_RANGE;
    if (!mul_ok(s_cap, g.H, &cap_rows) || !mul_ok(cap_rows, g.Db, &plane_bytes))
        return KVX_E_RANGE;
    for (int32_t q = 0; q < g.Q; ++q) {
        if (hf[q] == nullptr) {
            if (plane_bytes == 0) continue;      // an empty plane (s_cap = 0) may be NULL
            return KVX_E_NULL;
        }
        if (!aligned16(hf[q])) return KVX_E_ALIGN;
    }
    return KVX_OK;
}

#define KVX_TRY(expr)                         \
    do {                                      \
        kvx_status _s = (expr);               \
        if (_s != KVX_OK) return _s;          \
    } while (0)

}  // namespace

namespace {

// One row a call touches: bytes [lo, hi) for batch token `tok`.
struct Span {
    uint64_t lo, hi;
    int64_t tok;
};

// A HOST copy of a batch's token CSR follows its contract: tok_off[0] = 0,
// never decreasing, tok_off[num_reqs] = total_tokens (KVX_E_SHAPE otherwise).
// Everything that indexes per-token arrays by tok_off checks this first.
kvx_status check_tok_off(const kvx_reqs* reqs) {
    const int32_t nr = reqs->num_reqs;
    if (nr == 0) return reqs->total_tokens == 0 ? KVX_OK : KVX_E_SHAPE;
    if (reqs->tok_off == nullptr) return KVX_E_NULL;
    if (reqs->tok_off[0] != 0 || reqs->tok_off[nr] != reqs->total_tokens) return KVX_E_SHAPE;
    for (int32_t r = 0; r < nr; ++r)
        if (reqs->tok_off[r + 1] < reqs->tok_off[r]) return KVX_E_SHAPE;
    return KVX_OK;
}

// Slot of every batch token in one pool side, or -1 where the call skips the
// token (page-table index or page id out of range, as the kernels decide).
kvx_status side_slots(const kvx_reqs* reqs, const kvx_pool* p, const kvx_table* t,
                      std::vector<int64_t>* slot) {
    if (p->planes == nullptr) return KVX_E_NULL;
    if (p->num_pages < 0 || p->page_size < 1) return KVX_E_SHAPE;
    if (t->num_ids < 0) return KVX_E_SHAPE;
    if (reqs->num_reqs > 0 && t->pg_off == nullptr) return KVX_E_NULL;
    if (t->num_ids > 0 && t->page_ids == nullptr) return KVX_E_NULL;
    KVX_TRY(check_tok_off(reqs));
    slot->assign(static_cast<size_t>(reqs->total_tokens), -1);
    for (int32_t r = 0; r < reqs->num_reqs; ++r) {
        const int64_t off = reqs->tok_off[r], n = reqs->tok_off[r + 1] - off;
        for (int64_t k = 0; k < n; ++k) {
            // the index pg_off[r] + k / page_size, range-checked before the
            // sum is formed (a plain integer: no pg_off value makes it wrap)
            const int64_t kp = k / p->page_size, pg = t->pg_off[r];
            if (pg < -kp || pg >= t->num_ids - kp) continue;
            const int64_t idx = pg + kp;
            const int64_t page = t->page_ids[idx];
            if (page < 0 || page >= p->num_pages) continue;
            (*slot)[static_cast<size_t>(off + k)] = page * p->page_size + k % p->page_size;
        }
    }
    return KVX_OK;
}

// Rows of the live tokens on one side (Q per token).
void side_spans(const Geom& g, const kvx_reqs* reqs, const kvx_pool* p,
                const std::vector<int64_t>& slot, const void* staging,
                const std::vector<char>& live, std::vector<Span>* out) {
    out->clear();
    for (int32_t r = 0; r < reqs->num_reqs; ++r) {
        const int64_t off = reqs->tok_off[r], n = reqs->tok_off[r + 1] - off;
        for (int64_t k = 0; k < n; ++k) {
            const int64_t tok = off + k;
            if (!live[static_cast<size_t>(tok)]) continue;
            for (int32_t q = 0; q < g.Q; ++q) {
                uint64_t lo;
                if (p != nullptr) {
                    const int64_t s = slot[static_cast<size_t>(tok)];
                    lo = reinterpret_cast<uint64_t>(p->planes[q]) +
                         static_cast<uint64_t>(s / p->page_size) *
                             static_cast<uint64_t>(page_stride_of(p)) +
                         static_cast<uint64_t>(s % p->page_size) *
                             static_cast<uint64_t>(p->slot_stride);
                }
                else
                    lo = reinterpret_cast<uint64_t>(staging) +
                         static_cast<uint64_t>((off * g.Q + q * n + k) * g.R);
                out->push_back(Span{lo, lo + static_cast<uint64_t>(g.R), tok});
            }
        }
    }
}

bool by_lo(const Span& a, const Span& b) { return a.lo < b.lo || (a.lo == b.lo && a.tok < b.tok); }

// Written spans pairwise disjoint (else KVX_E_DUPLICATE), then no written span
// sharing a byte with a read span (else KVX_E_OVERLAP); *bad receives the
// batch token of an offending written span.  Sorts both vectors.
kvx_status spans_disjoint(std::vector<Span>* w, std::vector<Span>* rd, int64_t* bad) {
    std::sort(w->begin(), w->end(), by_lo);
    uint64_t hi = 0;
    for (const Span& x : *w) {
        if (x.lo < hi) {
            if (bad != nullptr) *bad = x.tok;
            return KVX_E_DUPLICATE;
        }
        hi = x.hi;
    }
    std::sort(rd->begin(), rd->end(), by_lo);
    std::vector<uint64_t> max_hi(rd->size());
    uint64_t m = 0;
    for (size_t i = 0; i < rd->size(); ++i) max_hi[i] = m = std::max(m, (*rd)[i].hi);
    // a written span [lo, hi) meets a read span iff some read span starting
    // before hi ends after lo
    for (const Span& x : *w) {
        const size_t i = static_cast<size_t>(
            std::lower_bound(rd->begin(), rd->end(), x.hi,
                             [](const Span& a, uint64_t v) { return a.lo < v; }) -
            rd->begin());
        if (i > 0 && max_hi[i - 1] > x.lo) {
            if (bad != nullptr) *bad = x.tok;
            return KVX_E_OVERLAP;
        }
    }
    return KVX_OK;
}

// Head rows of the live tokens on one side of a head-sliced copy: for each
// plane and each of the nh heads of the slice, Db bytes at the address the
// kernels use (NHD or HND blocks, slice starting at h->head0).
void head_spans(const Geom& g, const kvx_reqs* reqs, const kvx_pool* p, const kvx_heads* h,
                const std::vector<int64_t>& slot, const std::vector<char>& live,
                std::vector<Span>* out) {
    out->clear();
    const uint64_t B = static_cast<uint64_t>(p->page_size);
    const uint64_t stride = static_cast<uint64_t>(p->slot_stride);
    const uint64_t Db = static_cast<uint64_t>(g.Db);
    for (int64_t tok = 0; tok < reqs->total_tokens; ++tok) {
        if (!live[static_cast<size_t>(tok)]) continue;
        const uint64_t s = static_cast<uint64_t>(slot[static_cast<size_t>(tok)]);
        const uint64_t page = s / B, row = s % B;
        for (int32_t q = 0; q < g.Q; ++q)
            for (int32_t j = 0; j < g.H; ++j) {
                const uint64_t hd = static_cast<uint64_t>(h->head0 + j);
                const uint64_t off = h->block_layout == KVX_HND
                                         ? page * B * stride + (hd * B + row) * Db
                                         : (page * B + row) * stride + hd * Db;
                const uint64_t lo = reinterpret_cast<uint64_t>(p->planes[q]) + off;
                out->push_back(Span{lo, lo + Db, tok});
            }
    }
}

}  // namespace

namespace {

// KVX_VALIDATE=1 (debug): before enqueueing, every data-movement call
// synchronizes its stream, copies its tables to the host and checks the
// preconditions the kernels assume: written rows pairwise disjoint and, for
// the row ops, disjoint from the rows read.  Out-of-range ids stay legal
// (those rows are skipped and counted).  It costs a synchronization and
// O(Q * tokens) host work per call, so it is for debugging, not production;
// it cannot run on a stream under graph capture (KVX_E_HIP).
bool validate_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("KVX_VALIDATE");
        return e != nullptr && e[0] == '1';
    }();
    return on;
}

template <class T>
kvx_status to_host(const T* d, int64_t n, std::vector<T>* h) {
    h->assign(static_cast<size_t>(n), T());
    if (n == 0) return KVX_OK;
    if (d == nullptr) return KVX_E_NULL;
    return hipMemcpy(h->data(), d, sizeof(T) * static_cast<size_t>(n), hipMemcpyDeviceToHost) ==
                   hipSuccess
               ? KVX_OK
               : KVX_E_HIP;
}

struct HostTable {
    std::vector<int64_t> pg;
    std::vector<int32_t> ids;
    kvx_table t;
};

kvx_status host_table(const kvx_table* t, int32_t nr, HostTable* h) {
    KVX_TRY(to_host(t->pg_off, static_cast<int64_t>(nr) + 1, &h->pg));
    KVX_TRY(to_host(t->page_ids, t->num_ids, &h->ids));
    h->t = kvx_table{h->pg.data(), h->ids.data(), t->num_ids};
    return KVX_OK;
}

// Head-sliced copies: the head rows the call writes pairwise disjoint and
// none of them overlapping a head row it reads (tokens out of range on
// either side are left out, as the kernels skip them).
kvx_status heads_disjoint(const kvx_layout* layout, const kvx_reqs* r, const kvx_pool* src,
                          const kvx_table* st, const kvx_heads* sh, const kvx_pool* dst,
                          const kvx_table* dt, const kvx_heads* dh, int64_t* bad) {
    Geom g;
    KVX_TRY(check_layout(layout, &g));
    std::vector<int64_t> ss, ds;
    KVX_TRY(side_slots(r, src, st, &ss));
    KVX_TRY(side_slots(r, dst, dt, &ds));
    std::vector<char> live(static_cast<size_t>(r->total_tokens), 1);
    for (int64_t t = 0; t < r->total_tokens; ++t)
        if (ss[static_cast<size_t>(t)] < 0 || ds[static_cast<size_t>(t)] < 0)
            live[static_cast<size_t>(t)] = 0;
    std::vector<Span> w, rd;
    head_spans(g, r, dst, dh, ds, live, &w);
    head_spans(g, r, src, sh, ss, live, &rd);
    return spans_disjoint(&w, &rd, bad);
}

kvx_status validate_call(const kvx_layout* layout, const kvx_reqs* reqs, const kvx_pool* src,
                         const kvx_table* st, const kvx_pool* dst, const kvx_table* dt,
                         const void* staging, int64_t staging_bytes, const kvx_heads* sh,
                         const kvx_heads* dh, hipStream_t stream) {
    if (reqs->num_reqs == 0 || reqs->total_tokens == 0) return KVX_OK;
    if (hipStreamSynchronize(stream) != hipSuccess) return KVX_E_HIP;
    std::vector<int64_t> tok;
    KVX_TRY(to_host(reqs->tok_off, static_cast<int64_t>(reqs->num_reqs) + 1, &tok));
    const kvx_reqs hr{reqs->num_reqs, reqs->total_tokens, tok.data()};
    HostTable hs, hd;
    if (src != nullptr) KVX_TRY(host_table(st, reqs->num_reqs, &hs));
    if (dst != nullptr) KVX_TRY(host_table(dt, reqs->num_reqs, &hd));
    int64_t bad = -1;
    kvx_status s = check_tok_off(&hr);
    if (s == KVX_OK)
        s = sh != nullptr
                ? heads_disjoint(layout, &hr, src, &hs.t, sh, dst, &hd.t, dh, &bad)
                : kvx_check_disjoint(layout, &hr, src, src != nullptr ? &hs.t : nullptr, dst,
                                     dst != nullptr ? &hd.t : nullptr, staging, staging_bytes,
                                     &bad);
    if (s != KVX_OK)
        std::fprintf(stderr, "kvx: KVX_VALIDATE: %s (batch token %lld); nothing enqueued\n",
                     kvx_status_str(s), static_cast<long long>(bad));
    return s;
}

}  // namespace

extern "C" {

kvx_status kvx_gather(const kvx_layout* layout, const kvx_pool* src, const kvx_table* src_table,
                      const kvx_reqs* reqs, void* staging, int64_t staging_bytes,
                      unsigned long long* skipped, uint32_t flags, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_out_flags(flags));
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_reqs(reqs));
    KVX_TRY(check_pool(src, g));
    KVX_TRY(check_source_nonempty(src, reqs));
    KVX_TRY(check_table(src_table, reqs));
    KVX_TRY(check_staging(staging, staging_bytes, g, reqs));
    if (validate_enabled())
        KVX_TRY(validate_call(layout, reqs, src, src_table, nullptr, nullptr, staging,
                              staging_bytes, nullptr, nullptr, stream));
    return run_paged<PoolRef, StageRef>(0, g, reqs, src, src_table, nullptr, nullptr, nullptr,
                                        staging, skipped, stream,
                                        (flags & KVX_OUT_CACHED) ? 1u : 0u);
}

kvx_status kvx_scatter(const kvx_layout* layout, const void* staging, int64_t staging_bytes,
                       const kvx_reqs* reqs, const kvx_pool* dst, const kvx_table* dst_table,
                       unsigned long long* skipped, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_reqs(reqs));
    KVX_TRY(check_pool(dst, g));
    KVX_TRY(check_table(dst_table, reqs));
    KVX_TRY(check_staging(staging, staging_bytes, g, reqs));
    if (validate_enabled())
        KVX_TRY(validate_call(layout, reqs, nullptr, nullptr, dst, dst_table, staging,
                              staging_bytes, nullptr, nullptr, stream));
    return run_paged<StageRef, PoolRef>(1, g, reqs, nullptr, nullptr, const_cast<void*>(staging),
                                        dst, dst_table, nullptr, skipped, stream);
}

kvx_status kvx_gather_scatter(const kvx_layout* layout,
                              const kvx_pool* src, const kvx_table* src_table,
                              const kvx_reqs* reqs,
                              const kvx_pool* dst, const kvx_table* dst_table,
                              unsigned long long* skipped, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_reqs(reqs));
    KVX_TRY(check_pool(src, g));
    KVX_TRY(check_source_nonempty(src, reqs));
    KVX_TRY(check_table(src_table, reqs));
    KVX_TRY(check_pool(dst, g));
    KVX_TRY(check_table(dst_table, reqs));
    if (validate_enabled())
        KVX_TRY(validate_call(layout, reqs, src, src_table, dst, dst_table, nullptr, 0, nullptr,
                              nullptr, stream));
    return run_paged<PoolRef, PoolRef>(2, g, reqs, src, src_table, nullptr, dst, dst_table,
                                       nullptr, skipped, stream);
}

kvx_status kvx_gather_scatter_heads(const kvx_layout* layout,
                                    const kvx_pool* src, const kvx_table* src_table,
                                    const kvx_heads* src_heads,
                                    const kvx_reqs* reqs,
                                    const kvx_pool* dst, const kvx_table* dst_table,
                                    const kvx_heads* dst_heads,
                                    unsigned long long* skipped, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_layout(layout, &g));
    if (g.Db % 16 != 0) return KVX_E_ALIGN;
    KVX_TRY(check_reqs(reqs));
    KVX_TRY(check_pool(src, g));
    KVX_TRY(check_source_nonempty(src, reqs));
    KVX_TRY(check_table(src_table, reqs));
    KVX_TRY(check_heads(src_heads, src, g));
    KVX_TRY(check_pool(dst, g));
    KVX_TRY(check_table(dst_table, reqs));
    KVX_TRY(check_heads(dst_heads, dst, g));
    if (validate_enabled())
        KVX_TRY(validate_call(layout, reqs, src, src_table, dst, dst_table, nullptr, 0,
                              src_heads, dst_heads, stream));
    return run_heads(g, reqs, src, src_table, src_heads, dst, dst_table, dst_heads, skipped,
                     stream);
}

kvx_status kvx_extract_permute(const kvx_layout* layout, const void* const* hf_planes,
                               int64_t s_cap, int64_t seq_len, void* out, int64_t out_bytes,
                               uint32_t flags, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_out_flags(flags));
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_hf(g, hf_planes, s_cap, seq_len));
    int64_t need = 0;
    if (!mul_ok(seq_len, static_cast<int64_t>(g.Q) * g.R, &need)) return KVX_E_RANGE;
    if (need > 0 && out == nullptr) return KVX_E_NULL;
    if (!aligned16(out)) return KVX_E_ALIGN;
    if (out_bytes < need) return KVX_E_SHAPE;
    return run_permute<false>(g, const_cast<void* const*>(hf_planes), s_cap, seq_len, out,
                              (flags & KVX_OUT_CACHED) ? 1u : 0u, stream);
}

kvx_status kvx_rebuild_permute(const kvx_layout* layout, const void* in, int64_t in_bytes,
                               int64_t seq_len, void* const* hf_planes, int64_t s_cap,
                               uint32_t flags, hipStream_t stream) {
    Geom g;
    KVX_TRY(check_out_flags(flags));
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_hf(g, hf_planes, s_cap, seq_len));
    int64_t need = 0;
    if (!mul_ok(seq_len, static_cast<int64_t>(g.Q) * g.R, &need)) return KVX_E_RANGE;
    if (need > 0 && in == nullptr) return KVX_E_NULL;
    if (!aligned16(in)) return KVX_E_ALIGN;
    if (in_bytes < need) return KVX_E_SHAPE;
    return run_permute<true>(g, hf_planes, s_cap, seq_len, const_cast<void*>(in),
                             (flags & KVX_OUT_CACHED) ? 1u : 0u, stream);
}

kvx_status kvx_check_tables(int32_t num_reqs, int64_t total_tokens, const int64_t* tok_off,
                            const int64_t* pg_off, const int32_t* page_ids, int64_t num_ids,
                            int64_t num_pages, int32_t page_size, int32_t as_destination,
                            int64_t* bad_token) {
    if (bad_token != nullptr) *bad_token = -1;
    if (num_reqs < 0 || total_tokens < 0 || num_ids < 0 || num_pages < 0 || page_size < 1)
        return KVX_E_SHAPE;
    if (num_reqs > 0 && (tok_off == nullptr || pg_off == nullptr)) return KVX_E_NULL;
    if (num_ids > 0 && page_ids == nullptr) return KVX_E_NULL;
    if (num_reqs == 0) return total_tokens == 0 ? KVX_OK : KVX_E_SHAPE;
    if (tok_off[0] != 0 || tok_off[num_reqs] != total_tokens || pg_off[0] < 0)
        return KVX_E_SHAPE;
    int64_t slots = 0;
    if (!mul_ok(num_pages, page_size, &slots)) return KVX_E_RANGE;
    std::vector<uint64_t> seen;
    if (as_destination) seen.assign(static_cast<size_t>((slots + 63) / 64), 0);
    for (int32_t r = 0; r < num_reqs; ++r) {
        // compared before they are subtracted: tok_off[r] and pg_off[r] are
        // >= 0 here (checked at r - 1), so neither difference can overflow
        if (tok_off[r + 1] < tok_off[r] || pg_off[r + 1] < pg_off[r] || pg_off[r + 1] > num_ids) {
            if (bad_token != nullptr) *bad_token = tok_off[r];
            return KVX_E_SHAPE;
        }
        const int64_t n = tok_off[r + 1] - tok_off[r];
        const int64_t pages = pg_off[r + 1] - pg_off[r];
        if (pages < n / page_size + (n % page_size != 0 ? 1 : 0)) {
            if (bad_token != nullptr) *bad_token = tok_off[r];
            return KVX_E_SHAPE;
        }
        for (int64_t t = 0; t < n; ++t) {
            const int64_t page = page_ids[pg_off[r] + t / page_size];
            if (page < 0 || page >= num_pages) {
                if (bad_token != nullptr) *bad_token = tok_off[r] + t;
                return KVX_E_RANGE;
            }
            if (as_destination) {
                const int64_t slot = page * page_size + t % page_size;
                uint64_t& w = seen[static_cast<size_t>(slot / 64)];
                const uint64_t bit = uint64_t(1) << (slot % 64);
                if (w & bit) {
                    if (bad_token != nullptr) *bad_token = tok_off[r] + t;
                    return KVX_E_DUPLICATE;
                }
                w |= bit;
            }
        }
    }
    return KVX_OK;
}

kvx_status kvx_check_disjoint(const kvx_layout* layout, const kvx_reqs* reqs,
                              const kvx_pool* src, const kvx_table* src_table,
                              const kvx_pool* dst, const kvx_table* dst_table,
                              const void* staging, int64_t staging_bytes,
                              int64_t* bad_token) {
    if (bad_token != nullptr) *bad_token = -1;
    Geom g;
    KVX_TRY(check_layout(layout, &g));
    KVX_TRY(check_reqs(reqs));
    KVX_TRY(check_tok_off(reqs));
    if ((src == nullptr) != (src_table == nullptr) || (dst == nullptr) != (dst_table == nullptr))
        return KVX_E_NULL;
    if (src == nullptr && dst == nullptr) return KVX_E_UNSUPPORTED;
    const int64_t T = reqs->total_tokens;
    if (src == nullptr || dst == nullptr) {
        int64_t need = 0;
        if (!mul_ok(T, static_cast<int64_t>(g.Q) * g.R, &need)) return KVX_E_RANGE;
        if (need > 0 && staging == nullptr) return KVX_E_NULL;
        if (staging_bytes < need) return KVX_E_SHAPE;
    }
    std::vector<int64_t> ss, ds;
    if (src != nullptr) KVX_TRY(side_slots(reqs, src, src_table, &ss));
    if (dst != nullptr) KVX_TRY(side_slots(reqs, dst, dst_table, &ds));
    std::vector<char> live(static_cast<size_t>(T), 1);
    for (int64_t t = 0; t < T; ++t)
        if ((src != nullptr && ss[static_cast<size_t>(t)] < 0) ||
            (dst != nullptr && ds[static_cast<size_t>(t)] < 0))
            live[static_cast<size_t>(t)] = 0;
    std::vector<Span> w, rd;
    side_spans(g, reqs, dst, ds, staging, live, &w);
    side_spans(g, reqs, src, ss, staging, live, &rd);
    return spans_disjoint(&w, &rd, bad_token);
}

const char* kvx_status_str(int32_t status) {
    switch (status) {
        case KVX_OK: return "KVX_OK";
        case KVX_E_NULL: return "KVX_E_NULL: a required pointer is NULL";
        case KVX_E_SHAPE: return "KVX_E_SHAPE: counts or sizes are negative, inconsistent or too small";
        case KVX_E_ALIGN: return "KVX_E_ALIGN: a base, stride, buffer or row size is not a multiple of 16 bytes";
        case KVX_E_DTYPE: return "KVX_E_DTYPE: unknown dtype code";
        case KVX_E_RANGE: return "KVX_E_RANGE: a size exceeds what one call supports";
        case KVX_E_UNSUPPORTED: return "KVX_E_UNSUPPORTED: not implemented by this build";
        case KVX_E_HIP: return "KVX_E_HIP: the HIP runtime refused a launch or a device query";
        case KVX_E_DUPLICATE: return "KVX_E_DUPLICATE: two written rows are the same row or overlap";
        case KVX_E_OVERLAP: return "KVX_E_OVERLAP: a written row overlaps a row the call reads";
        default: return "unknown kvx_status";
    }
}

int32_t kvx_abi_version(void) { return KVX_ABI_VERSION; }

}  // extern "C"
