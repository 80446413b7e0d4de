// Row gather / scatter along a token order: the explicit reorder pass that
// brings rows into Hilbert (or tile) sequence order and back
// ("Hilbert-Guided Sparse Local Attention": tokens reordered along the curve,
// windows formed on the reordered sequence, the path computed once and
// cached).  Pure HBM copy: every row is read once and written once, in
// 16-byte vectors when the row length allows it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "na_internal.h"

namespace {

// One (batch, head) slice per grid row (grid-stride over slices), a block of
// 256 threads covers 256 >> vshift whole rows (1 << vshift vectors per row),
// grid-stride over the slice's rows: no 64-bit division per vector.
template <typename V>
__global__ __launch_bounds__(256) void permute_rows(const char* __restrict__ in, char* __restrict__ out,
                                                    int64_t N, int64_t heads, int64_t slices, int vshift,
                                                    int64_t in_sb, int64_t in_sh, int64_t in_sn,
                                                    int64_t out_sb, int64_t out_sh, int64_t out_sn,
                                                    const int32_t* __restrict__ perm, int inverse) {
    const int vi = threadIdx.x & ((1 << vshift) - 1);
    const int rpb = 256 >> vshift;                         // rows per block
    const int64_t r0 = (int64_t)blockIdx.x * rpb + (threadIdx.x >> vshift);
    const int64_t rstep = (int64_t)gridDim.x * rpb;
    for (int64_t bh = blockIdx.y; bh < slices; bh += gridDim.y) {
        const int64_t b = bh / heads, h = bh % heads;      // uniform
        const char* ib = in + b * in_sb + h * in_sh + vi * (int64_t)sizeof(V);
        char* ob = out + b * out_sb + h * out_sh + vi * (int64_t)sizeof(V);
        for (int64_t pos = r0; pos < N; pos += rstep) {
            const int64_t tok = perm[pos];
            const int64_t src = inverse ? pos : tok;
            const int64_t dst = inverse ? tok : pos;
            *(V*)(ob + dst * out_sn) = *(const V*)(ib + src * in_sn);
        }
    }
}

}  // namespace

int na_permute_launch(const void* in, void* out, int64_t B, int64_t H, int64_t N, int64_t row_bytes,
                      int64_t in_sb, int64_t in_sh, int64_t in_sn, int64_t out_sb, int64_t out_sh,
                      int64_t out_sn, const int32_t* perm, int inverse, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const bool wide = row_bytes % 16 == 0 && in_sb % 16 == 0 && in_sh % 16 == 0 &&
                      in_sn % 16 == 0 && out_sb % 16 == 0 && out_sh % 16 == 0 &&
                      out_sn % 16 == 0 && ((uintptr_t)in % 16) == 0 && ((uintptr_t)out % 16) == 0;
    const int64_t vbytes = wide ? 16 : 4;
    const int64_t vec_per_row = row_bytes / vbytes;
    // rows are whole vectors, a power of two of them, at most one block's worth
    if (row_bytes % vbytes != 0 || vec_per_row < 1 || vec_per_row > 256 ||
        (vec_per_row & (vec_per_row - 1)) != 0)
        return (int)hipErrorInvalidValue;
    const int64_t slices = B * H;
    if (slices == 0 || N == 0) return 0;
    int vshift = 0;
    while ((int64_t(1) << vshift) < vec_per_row) ++vshift;
    const int64_t rpb = 256 >> vshift;
    int64_t bx = (N + rpb - 1) / rpb;
    const int64_t by = slices < 65535 ? slices : 65535;
    // about 16 blocks per CU in all; the rest is grid-stride
    const int64_t cap = (4096 + by - 1) / by;
    if (bx > cap) bx = cap;
    const dim3 grid((unsigned)bx, (unsigned)by);
    if (wide)
        hipLaunchKernelGGL(permute_rows<uint4>, grid, dim3(256), 0, st, (const char*)in, (char*)out,
                           N, H, slices, vshift, in_sb, in_sh, in_sn, out_sb, out_sh, out_sn, perm,
                           inverse);
    else
        hipLaunchKernelGGL(permute_rows<uint32_t>, grid, dim3(256), 0, st, (const char*)in,
                           (char*)out, N, H, slices, vshift, in_sb, in_sh, in_sn, out_sb, out_sh,
                           out_sn, perm, inverse);
    return (int)hipGetLastError();
}
