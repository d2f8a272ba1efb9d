// read_probe.hip -- a plain read kernel that measures the HBM read rate the decode kernels can hope
// for: 2 KiB tiles (the cache's (block, KV head) tile) streamed by about 2048 waves with 16-byte
// non-temporal loads, in a given tile order (sequential, or shuffled like a paged block table).
// A benchmark aid beside libkvq.so, not part of the cache's ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 2048;     // bytes per tile
constexpr int kInFlight = 4;    // tiles loaded before any is consumed

// Wave w reads tiles order[i] for i in [w * n / nw, (w + 1) * n / nw): each lane 32 bytes of each
// tile (two 16-byte loads), kInFlight tiles at a time.  The XOR of everything read goes to
// sink[w * 64 + lane], so no load is dead.
__global__ __launch_bounds__(64) void read_tiles(const uint8_t* base, const int32_t* order, int n,
                                                 uint32_t* sink) {
    const int lane = threadIdx.x;
    const int nw = gridDim.x;
    const int w = blockIdx.x;
    const int i0 = (int)((int64_t)w * n / nw), i1 = (int)((int64_t)(w + 1) * n / nw);
    u32x4 x = {0u, 0u, 0u, 0u};
    int i = i0;
    for (; i + kInFlight <= i1; i += kInFlight) {
        u32x4 a[kInFlight], b[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const uint8_t* t = base + (size_t)order[i + j] * kTile + 16 * lane;
            a[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t));
            b[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + 1024));
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) x ^= a[j] ^ b[j];
    }
    for (; i < i1; ++i) {
        const uint8_t* t = base + (size_t)order[i] * kTile + 16 * lane;
        x ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t));
        x ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(t + 1024));
    }
    sink[(size_t)w * 64 + lane] = x.x ^ x.y ^ x.z ^ x.w;
}

}  // namespace

// Read n 2 KiB tiles of `base` (device memory of at least (max order + 1) * 2048 bytes) in the
// order given by `order` (device int32 [n]) with `waves` waves; `sink` is device uint32
// [waves * 64].  Returns 0, or -1 for bad arguments, or the HIP error code at launch.
extern "C" int kvq_probe_read_tiles(const void* base, const int32_t* order, int32_t n, int32_t waves,
                                    uint32_t* sink, void* stream) {
    if (!base || !order || !sink || n <= 0 || waves <= 0) return -1;
    read_tiles<<<dim3((unsigned)waves), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint8_t*>(base), order, n, sink);
    return (int)hipGetLastError();
}
