// Attainable HBM read bandwidth on one MI355X: a plain streaming read, the
// ceiling a kernel that reads each KV row once can approach.  Not part of the
// decode path; the benchmark uses it to put the decode kernels' bandwidth
// next to what plain reads achieve on the same part.
//
// Plain reads: each thread reads 16-byte chunks with nontemporal loads (the
// data is used once), kUnroll chunks in flight per loop trip, grid-stride
// over the buffer, and folds them into a register.  The register is stored
// only if it equals a value no real buffer produces, so the loads cannot be
// optimised away and the kernel writes (in practice) nothing.
//
// Direct-to-LDS reads: the path the decode kernels stage their KV tiles
// through (global_load_lds_dwordx4, 1 KB per wave instruction, no register
// round trip).  `active` waves of each 256-thread workgroup stream
// interleaved 1 KB pieces into a private 16-slot LDS ring, at most 16 in
// flight per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void hbm_stream_read_kernel(
    const u32x4 *__restrict__ src, long long n16, unsigned *__restrict__ sink)
{
    u32x4 acc = {0u, 0u, 0u, 0u};
    const long long stride = (long long)gridDim.x * kThreads;
    long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u];
    }
    for (; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(src + i);
    const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u)
        sink[blockIdx.x] = x;
}

__global__ __launch_bounds__(kThreads) void hbm_stream_read_lds_kernel(
    const uint8_t *__restrict__ src, long long n_pieces, int active)
{
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * 16 * 1024];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (w >= active)
        return;
    const long long waves = (long long)gridDim.x * active;
    int slot = 0;
    for (long long k = (long long)blockIdx.x * active + w; k < n_pieces; k += waves) {
        const unsigned m0 = __builtin_amdgcn_readfirstlane(
            (unsigned)(uintptr_t)(ring + w * 16384 + (slot & 15) * 1024));
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(m0), "v"(src + k * 1024 + lane * 16)
                     : "memory", "m0");
        // a slot is written again 16 loads later, after its load has landed
        if ((++slot & 7) == 0)
            __builtin_amdgcn_s_waitcnt((8 & 15) | (0x7 << 4) | (0xF << 8));   // vmcnt(8)
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));                     // vmcnt(0)
}

// Request rate of one CU when the data sits in L2: `active` waves of each
// workgroup read 1 KB pieces of a 256 KB window (window blockIdx & 7, so each
// XCD's L2 holds the eight windows after the first pass), 8 pieces per batch
// with the previous batch still in flight, either direct-to-LDS (kLds) or
// into registers.  What it measures is how fast a CU accepts and completes
// 16-byte-per-lane requests that hit L2, the ceiling of a tile-load burst.
template <bool kLds>
__global__ __launch_bounds__(kThreads) void l2_request_rate_kernel(
    const uint8_t *__restrict__ src, int n_batches, int active, unsigned *__restrict__ sink)
{
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * 16 * 1024];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (w >= active)
        return;
    const uint8_t *win = src + (size_t)(blockIdx.x & 7) * 256 * 1024 + lane * 16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int k = 0; k < n_batches; ++k) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const unsigned piece = (unsigned)(k * 8 + u + w * 64) & 255u;
            if (kLds) {
                const unsigned m0 = __builtin_amdgcn_readfirstlane(
                    (unsigned)(uintptr_t)(ring + w * 16384 + ((k & 1) * 8 + u) * 1024));
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                             :
                             : "s"(m0), "v"(win + piece * 1024)
                             : "memory", "m0");
            } else {
                v[u] = *(const u32x4 *)(win + piece * 1024);
            }
        }
        if (kLds) {
            __builtin_amdgcn_s_waitcnt((8 & 15) | (0x7 << 4) | (0xF << 8));   // vmcnt(8)
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc ^= v[u];
        }
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));                     // vmcnt(0)
    const unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ ring[w * 16384 + lane];
    if (x == 0x9E3779B9u)
        sink[blockIdx.x] = x;
}

} // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) at `src` once, with
// `grid` workgroups of 256 threads; `sink` must hold `grid` unsigned words.
// Returns 0 after enqueuing on `stream`, 1 for bad arguments, 2 if the launch
// failed.
int hbm_stream_read(const void *src, size_t bytes, unsigned *sink, int grid, hipStream_t stream)
{
    if (!src || !sink || grid < 1 || (bytes & 15) || ((uintptr_t)src & 15))
        return 1;
    hipLaunchKernelGGL(hbm_stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const u32x4 *)src, (long long)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Read `bytes` (a multiple of 1024, 16-byte aligned) at `src` once into LDS
// with direct-to-LDS loads: `grid` workgroups, `active` (1 .. 4) streaming
// waves each.  Returns 0 after enqueuing on `stream`, 1 for bad arguments, 2
// if the launch failed.
int hbm_stream_read_lds(const void *src, size_t bytes, int grid, int active, hipStream_t stream)
{
    if (!src || grid < 1 || active < 1 || active > 4 || (bytes & 1023) || ((uintptr_t)src & 15))
        return 1;
    hipLaunchKernelGGL(hbm_stream_read_lds_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       (const uint8_t *)src, (long long)(bytes / 1024), active);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// L2-resident request rate: `grid` workgroups, `active` (1 .. 4) waves each,
// every wave reading 8 * n_batches pieces of 1 KB from a 256 KB window of
// `src` (which must hold 8 such windows: 2 MiB, 16-byte aligned);
// direct-to-LDS when `lds` is nonzero, else into registers.  `sink` must
// hold `grid` unsigned words.  Returns 0 after enqueuing on `stream`, 1 for
// bad arguments, 2 if the launch failed.
int l2_request_rate(const void *src, int n_batches, int grid, int active, int lds, unsigned *sink,
                    hipStream_t stream)
{
    if (!src || !sink || grid < 1 || n_batches < 1 || active < 1 || active > 4 ||
        ((uintptr_t)src & 15))
        return 1;
    if (lds)
        hipLaunchKernelGGL(l2_request_rate_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, (const uint8_t *)src, n_batches, active, sink);
    else
        hipLaunchKernelGGL(l2_request_rate_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, (const uint8_t *)src, n_batches, active, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

} // extern "C"
