// How fast can a kernel stream reads from HBM on this GPU?  The decode
// kernel reads K and V once and is bound by that rate, so its roofline
// fraction is best read against what plain streaming reads reach, not
// only against the nameplate 8 TB/s.
//
// A 4 GiB buffer is read once per launch with 16-byte vector loads, U loads
// in flight per thread, in two layouts:
//   grid-stride  -- consecutive threads read consecutive 16-byte pieces, the
//                   whole grid sweeps the buffer U pieces per thread at a time;
//   block-span   -- each workgroup reads one contiguous span (1/grid of the
//                   buffer) with its threads striding inside it, the layout of
//                   a workgroup streaming its own K/V range.
// Each thread folds what it read into one word (so the loads are not
// removed) and writes that word; the writes are 0.1 % of the bytes.  Every
// configuration runs 3 untimed and 10 timed launches between HIP events;
// the report gives the best and the median rate in TB/s (10^12 B/s).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Pieces i, i + nth, ..., i + (U-1) nth per step; every index stays below n16.
template <int U>
__global__ __launch_bounds__(512) void read_grid_stride(const u32x4* __restrict__ p, uint64_t n16, uint32_t* out) {
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t nth = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    uint64_t i = tid;
    for (; i + (U - 1) * nth < n16; i += U * nth) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * nth];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += nth) acc ^= fold(p[i]);
    out[tid] = acc;
}

// Workgroup b reads pieces [b*span, min((b+1)*span, n16)).
template <int U>
__global__ __launch_bounds__(512) void read_block_span(const u32x4* __restrict__ p, uint64_t n16, uint32_t* out) {
    const uint64_t span = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = (uint64_t)blockIdx.x * span;
    const uint64_t hi = std::min<uint64_t>(lo + span, n16);
    const uint64_t nt = blockDim.x;
    uint32_t acc = 0;
    uint64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * nt < hi; i += U * nt) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * nt];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (; i < hi; i += nt) acc ^= fold(p[i]);
    out[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

typedef void (*Kern)(const u32x4*, uint64_t, uint32_t*);

static void run(const char* name, Kern k, int grid, int block, const u32x4* buf, uint64_t n16, uint32_t* out) {
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int r = 0; r < 3; ++r) k<<<grid, block>>>(buf, n16, out);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<float> ms;
    for (int r = 0; r < 10; ++r) {
        CHECK(hipEventRecord(e0));
        k<<<grid, block>>>(buf, n16, out);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float t = 0;
        CHECK(hipEventElapsedTime(&t, e0, e1));
        ms.push_back(t);
    }
    std::sort(ms.begin(), ms.end());
    const double bytes = (double)n16 * 16.0;
    printf("| %s | %d x %d | %.3f | %.2f | %.2f |\n", name, grid, block, ms[0], bytes / (ms[0] * 1e-3) / 1e12,
           bytes / (ms[5] * 1e-3) / 1e12);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
}

int main() {
    const uint64_t bytes = 4ull << 30;
    const uint64_t n16 = bytes / 16;
    u32x4* buf = nullptr;
    uint32_t* out = nullptr;
    CHECK(hipMalloc(&buf, bytes));
    CHECK(hipMemset(buf, 0x5a, bytes));
    const int max_threads = 8192 * 512;
    CHECK(hipMalloc(&out, (size_t)max_threads * sizeof(uint32_t)));
    CHECK(hipDeviceSynchronize());
    printf("Streaming reads of a 4 GiB buffer, 16-byte loads; TB/s = 10^12 B/s\n\n");
    printf("| layout, loads in flight per thread | grid x block | best ms | best TB/s | median TB/s |\n");
    printf("|---|---|---|---|---|\n");
    const int grids[] = {256, 512, 1024, 2048, 4096, 8192};
    for (int grid : grids) {
        run("grid-stride, U=4", read_grid_stride<4>, grid, 256, buf, n16, out);
        run("grid-stride, U=8", read_grid_stride<8>, grid, 256, buf, n16, out);
    }
    for (int grid : grids) {
        run("block-span, U=4", read_block_span<4>, grid, 256, buf, n16, out);
        run("block-span, U=8", read_block_span<8>, grid, 256, buf, n16, out);
    }
    run("grid-stride, U=8", read_grid_stride<8>, 1024, 512, buf, n16, out);
    run("block-span, U=8", read_block_span<8>, 512, 512, buf, n16, out);
    run("block-span, U=8", read_block_span<8>, 1024, 512, buf, n16, out);
    CHECK(hipFree(out));
    CHECK(hipFree(buf));
    return 0;
}
