// Measurement reference for bench.py, not part of the rotate + quantize path
// and not linked into libhadarot.so: a plain streaming kernel that reads and
// writes given byte counts in one launch, 16 bytes per lane per access with
// the same streaming (non-temporal) loads and stores as the path's kernels.
// Timed like a part (same bytes, launches back to back over copies of the
// input), it gives the floor a kernel of that shape meets on this GPU with
// no arithmetic at all.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kPer = 4;   // 16-byte pieces per thread
constexpr int kThreads = 256;

// Thread t of block b handles pieces b * 1024 + t + 256 k (k < 4): it loads
// the ones below nr and stores the ones below nw (the XOR of what it loaded,
// so that no load is dead).
__global__ void __launch_bounds__(kThreads) stream_kernel(const u32x4_t* __restrict__ src, int64_t nr,
                                                          u32x4_t* __restrict__ dst, int64_t nw) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kPer + threadIdx.x;
    u32x4_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + static_cast<int64_t>(kThreads) * k;
        v[k] = i < nr ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
    u32x4_t acc = v[0];
#pragma unroll
    for (int k = 1; k < kPer; ++k) acc ^= v[k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i = base + static_cast<int64_t>(kThreads) * k;
        if (i < nw) __builtin_nontemporal_store(acc ^ v[k], dst + i);
    }
}
// Issue-rate probe: every thread runs eight independent float FMA chains
// for `iters` rounds.  With W waves per SIMD and nothing else running, a
// SIMD issues a wave64 FMA every 4 cycles, so the launch takes about
// W * iters * 8 * 4 cycles: its duration gives the shader clock the GPU ran
// at (it varies between GPUs of one model under power management).
__global__ void __launch_bounds__(kThreads) clock_kernel(float* out, int iters, float a) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], a, 0.5f);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
    if (s == 12345.0f) out[blockIdx.x] = s;   // keeps the chains live; practically never stored
}
}  // namespace

// Runs clock_kernel on `blocks` workgroups of 256 threads (out: at least
// `blocks` floats of device memory, practically never written).  Returns 0,
// -1 for invalid arguments, or -3 if the launch failed.
extern "C" int hr_clock_ref(float* out, int blocks, int iters, void* stream) {
    if (out == nullptr || blocks <= 0 || iters <= 0) return -1;
    hipLaunchKernelGGL(clock_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), out, iters, 0.999f);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Reads read_bytes from src and writes write_bytes to dst (both multiples of
// 16; pointers 16-byte aligned; device memory) in one launch on `stream`.
// Returns 0, -1 for invalid arguments, or -3 if the launch failed.
extern "C" int hr_stream_ref(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, void* stream) {
    if (read_bytes < 0 || write_bytes < 0 || (read_bytes | write_bytes) % 16 != 0 ||
        (read_bytes > 0 && (src == nullptr || reinterpret_cast<uintptr_t>(src) % 16 != 0)) ||
        (write_bytes > 0 && (dst == nullptr || reinterpret_cast<uintptr_t>(dst) % 16 != 0)))
        return -1;
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    const int64_t n = nr > nw ? nr : nw;
    if (n == 0) return 0;
    const int64_t grid = (n + kThreads * kPer - 1) / (kThreads * kPer);
    if (grid > 0x7FFFFFFF) return -1;
    hipLaunchKernelGGL(stream_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), nr,
                       static_cast<u32x4_t*>(dst), nw);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
