// HBM read-bandwidth probe for the benchmark's context figures (not part of the
// layer or its C ABI; built as its own small library, libmoe_probe.so).
//
// Every lane streams 16-byte loads over the buffer with a grid stride, four
// loads in flight per iteration, and folds them into one register; a lane
// writes only if that fold hits a value the caller chose never to occur, so the
// loads stay live and the writes are negligible.  The figure it gives is what a
// plain streaming read reaches on the part, the practical ceiling the
// HBM-bound kernels are compared with beside the nominal 8 TB/s.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_read_probe(const u32x4_t* __restrict__ p, long n16, uint32_t never,
                                                    uint32_t* __restrict__ out) {
    const long stride = (long)gridDim.x * 256;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        const u32x4_t b = __builtin_nontemporal_load(p + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) + (c[0] ^ c[1] ^ c[2] ^ c[3]) +
               (d[0] ^ d[1] ^ d[2] ^ d[3]);
    }
    for (; i < n16; i += stride) {
        const u32x4_t a = p[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    if (acc == never) out[blockIdx.x] = acc;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) at `p` once with `blocks`
// workgroups of 256 lanes; `out` must hold `blocks` uint32 (written only in
// the case above).  Returns 0, or -1 on bad arguments or a failed launch.
extern "C" int moe_probe_read(const void* p, size_t bytes, uint32_t never, uint32_t* out, int blocks, void* stream) {
    if (!p || !out || blocks <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(p) & 15)) return -1;
    hipLaunchKernelGGL(k_read_probe, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t*>(p), (long)(bytes / 16), never, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
