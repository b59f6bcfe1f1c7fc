// devfill.hip -- device side of the seeded input generators (not the kvx
// path; shares no code with it).
//
//   wl_fill_hash: 8-byte word i of the buffer gets output (ctr0 + i) of the
//     SplitMix64 generator started at `seed` (Steele, Lea & Flood, OOPSLA
//     2014): mix(seed + (ctr0 + i + 1) * 0x9E3779B97F4A7C15), the same words
//     workloads.splitmix64 computes on the host.
//   wl_copy: a plain 16-byte-per-lane copy of nbytes, used to calibrate HBM
//     byte counters (FETCH_SIZE / WRITE_SIZE) against a kernel of known
//     traffic.
//   wl_read_stream: a streaming HBM reader standing in for decode attention
//     reading its KV, to load the memory system while the kvx path runs.
//   wl_row_pattern: a table-free mover of rows that measures what the
//     paged ops' access patterns cost by themselves (random slots on either
//     side, no page tables read).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__global__ void k_fill_hash(uint64_t* __restrict__ dst, int64_t nwords, uint64_t seed,
                            uint64_t ctr0) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 2;
    for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 2;
         i < nwords; i += stride) {
        const uint64_t c = ctr0 + static_cast<uint64_t>(i);
        const uint64_t a = mix64(seed + (c + 1) * 0x9E3779B97F4A7C15ull);
        if (i + 1 < nwords) {
            const uint64_t b = mix64(seed + (c + 2) * 0x9E3779B97F4A7C15ull);
            *reinterpret_cast<ulonglong2*>(dst + i) = make_ulonglong2(a, b);
        } else {
            dst[i] = a;
        }
    }
}

__global__ void k_copy16(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += stride)
        dst[i] = src[i];
}

// A decode-like HBM reader: streams through the buffer with 16-byte loads and
// folds the words together; the fold is stored only if it equals a value the
// data practically never produces, so the loads cannot be dropped.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void k_read_stream(const u32x4* __restrict__ src, int64_t n16,
                              unsigned long long* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
         i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

// Row r of a pattern launch is row t = r % T of plane q = r / T.  Its place
// on a random side is slot ((t + set * T) * 40503 + q * 977) mod S of plane q
// in a [Q][S][R] buffer -- a bijection of the plane's S slots (S a power of
// two, the multiplier odd), so sets 0 .. S/T - 1 touch disjoint slots; on a
// contiguous side it is row q * T + t of a [Q][T][R] buffer.  Rows of R
// bytes (a multiple of 16, at most 4 KiB: lane l moves bytes 16 l + 1024 v
// of a row), K rows per wave, two-wave workgroups; loads and stores are
// 16-byte nontemporal, all K rows' loads issued before the first store.
struct PatternArgs {
    const char* src;
    char* dst;
    unsigned* sink;
    int32_t Q, T, S, set, R;
    uint32_t mode;              // 1 read, 2 write, 4 random source, 8 random destination
};

typedef __attribute__((address_space(1))) u32x4 g_u32x4;

__device__ __forceinline__ uint64_t pattern_row(uint64_t base, bool rnd, uint32_t q, uint32_t t,
                                                const PatternArgs& a) {
    if (rnd) {
        const uint32_t slot = ((t + static_cast<uint32_t>(a.set) * a.T) * 40503u + q * 977u) &
                              static_cast<uint32_t>(a.S - 1);
        return base + (static_cast<uint64_t>(q) * a.S + slot) * static_cast<uint64_t>(a.R);
    }
    return base + (static_cast<uint64_t>(q) * a.T + t) * static_cast<uint64_t>(a.R);
}

template <int K>
__global__ __launch_bounds__(128) void k_row_pattern(PatternArgs a) {
    constexpr int V = 4;                                   // 1 KiB steps of a row
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = blockIdx.x * 2u + (threadIdx.x >> 6);
    const uint32_t rows = static_cast<uint32_t>(a.Q) * static_cast<uint32_t>(a.T);
    const uint32_t R = static_cast<uint32_t>(a.R);
    uint64_t sa[K], da[K];
    u32x4 x[K][V];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const uint32_t r = w * K + j;
        const uint32_t q = r < rows ? r / a.T : 0u, t = r < rows ? r % a.T : 0u;
        sa[j] = pattern_row(reinterpret_cast<uint64_t>(a.src), a.mode & 4u, q, t, a);
        da[j] = pattern_row(reinterpret_cast<uint64_t>(a.dst), a.mode & 8u, q, t, a);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const uint32_t off = v * 1024u + lane * 16u;
            if ((a.mode & 1u) && off < R)
                x[j][v] = __builtin_nontemporal_load(reinterpret_cast<const g_u32x4*>(sa[j] + off));
            else
                x[j][v] = u32x4{w, lane, static_cast<uint32_t>(j), static_cast<uint32_t>(v)};
        }
    }
    if (a.mode & 2u) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (w * K + j < rows) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const uint32_t off = v * 1024u + lane * 16u;
                    if (off < R)
                        __builtin_nontemporal_store(x[j][v],
                                                    reinterpret_cast<g_u32x4*>(da[j] + off));
                }
            }
        }
    } else {
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < K; ++j)
#pragma unroll
            for (int v = 0; v < V; ++v) acc ^= x[j][v].x ^ x[j][v].w;
        if (acc == 0x9e3779b9u && lane == 0) a.sink[w & 2047u] = acc;   // keeps the loads
    }
}

int grid_for(int64_t items) {
    int64_t g = (items + 255) / 256;
    if (g > 65536) g = 65536;
    return g < 1 ? 1 : static_cast<int>(g);
}

}  // namespace

extern "C" {

// Returns 0 on success, -1 on bad arguments, else the hipError_t of the launch.
int wl_fill_hash(void* dst, int64_t nbytes, uint64_t seed, uint64_t ctr0, hipStream_t stream) {
    if (nbytes == 0) return 0;
    if (dst == nullptr || nbytes < 0 || nbytes % 8 != 0 ||
        (reinterpret_cast<uintptr_t>(dst) & 15u) != 0)
        return -1;
    const int64_t nwords = nbytes / 8;
    hipLaunchKernelGGL(k_fill_hash, dim3(grid_for((nwords + 1) / 2)), dim3(256), 0, stream,
                       static_cast<uint64_t*>(dst), nwords, seed, ctr0);
    return static_cast<int>(hipGetLastError());
}

int wl_copy(void* dst, const void* src, int64_t nbytes, hipStream_t stream) {
    if (nbytes == 0) return 0;
    if (dst == nullptr || src == nullptr || nbytes < 0 || nbytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(dst) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
        return -1;
    hipLaunchKernelGGL(k_copy16, dim3(grid_for(nbytes / 16)), dim3(256), 0, stream,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), nbytes / 16);
    return static_cast<int>(hipGetLastError());
}

// Reads nbytes (multiple of 16) of src once with `blocks` workgroups of 256
// threads (1..2048; fewer blocks, lighter load); sink must hold 2048 words.
int wl_read_stream(const void* src, int64_t nbytes, void* sink, int blocks, hipStream_t stream) {
    if (nbytes == 0) return 0;
    if (src == nullptr || sink == nullptr || nbytes < 0 || nbytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15u) != 0 || blocks < 1 || blocks > 2048)
        return -1;
    hipLaunchKernelGGL(k_read_stream, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), nbytes / 16,
                       static_cast<unsigned long long*>(sink));
    return static_cast<int>(hipGetLastError());
}

// Table-free row pattern (see k_row_pattern): Q planes of T rows of R bytes
// (16 .. 4096, a multiple of 16), S slots per plane on a random side (a power
// of two >= T), slot set `set` (0 .. S/T - 1), K rows per wave (1, 2 or 4),
// mode bits 1 read, 2 write, 4 random source, 8 random destination.
// src_bytes / dst_bytes must hold what the mode addresses ([Q][S][R] random,
// [Q][T][R] contiguous); sink must hold 2048 words.
int wl_row_pattern(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes, void* sink,
                   int32_t Q, int32_t T, int32_t S, int32_t R, int32_t K, int32_t set,
                   uint32_t mode, hipStream_t stream) {
    if (Q < 1 || T < 1 || S < T || (S & (S - 1)) != 0 || set < 0 ||
        static_cast<int64_t>(set + 1) * T > S || (K != 1 && K != 2 && K != 4) ||
        R < 16 || R > 4096 || R % 16 != 0 ||
        (mode & 3u) == 0 || mode > 15u || sink == nullptr ||
        static_cast<int64_t>(Q) * T > (int64_t(1) << 30))
        return -1;
    const int64_t rnd = static_cast<int64_t>(Q) * S * R, cont = static_cast<int64_t>(Q) * T * R;
    // the source is addressed in every mode (a write-only launch computes but never reads it)
    if (src == nullptr || src_bytes < ((mode & 4u) ? rnd : cont)) return -1;
    if ((mode & 2u) && (dst == nullptr || dst_bytes < ((mode & 8u) ? rnd : cont))) return -1;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0)
        return -1;
    PatternArgs a{static_cast<const char*>(src), static_cast<char*>(dst),
                  static_cast<unsigned*>(sink), Q, T, S, set, R, mode};
    const int64_t waves = (static_cast<int64_t>(Q) * T + K - 1) / K;
    const dim3 grid(static_cast<unsigned>((waves + 1) / 2));
    switch (K) {
        case 1: hipLaunchKernelGGL(k_row_pattern<1>, grid, dim3(128), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(k_row_pattern<2>, grid, dim3(128), 0, stream, a); break;
        default: hipLaunchKernelGGL(k_row_pattern<4>, grid, dim3(128), 0, stream, a); break;
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
