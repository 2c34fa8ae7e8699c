// Zero fills for gradients whose defining sums are empty: with no query rows
// the gradients of the keys and values, and of every weight, are sums over
// nothing.  Plain kernels rather than hipMemsetAsync, so the calls stay
// valid inside a captured HIP graph.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

// One thread per 16 bytes of a [B, H, L, 64] view: 64 features are 8 (bf16)
// or 16 (fp32) such pieces per row.
__global__ __launch_bounds__(256) void zero_view(char* p, long long s0, long long s1, long long s2, int H, int L,
                                                 int elem, long long pieces) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= pieces) return;
    const int per_row = 64 * elem / 16;
    const long long row = i / per_row;
    const int piece = (int)(i % per_row);
    const long long l = row % L, bh = row / L;
    const long long off = ((bh / H) * s0 + (bh % H) * s1 + l * s2) * elem + piece * 16;
    *reinterpret_cast<uint4*>(p + off) = make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void zero_f32(float* p, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero_view(void* p, const long long s[3], int B, int H, int L, int elem, hipStream_t st) {
    if (elem != 2 && elem != 4) return hipErrorInvalidValue;
    const long long pieces = (long long)B * H * L * (64 * elem / 16);
    if (pieces == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_view, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, static_cast<char*>(p),
                       s[0], s[1], s[2], H, L, elem, pieces);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, long long n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace mha
