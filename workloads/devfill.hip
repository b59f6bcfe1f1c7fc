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

}  // extern "C"
