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

template <typename V>
__global__ __launch_bounds__(256) void permute_rows(const char* __restrict__ in, char* __restrict__ out,
                                                    int64_t rows_per_head, int64_t heads,
                                                    int64_t vec_per_row, int64_t total_vec,
                                                    int64_t in_sb, int64_t in_sh, int64_t in_sn,
                                                    int64_t out_sb, int64_t out_sh, int64_t out_sn,
                                                    const int32_t* __restrict__ perm, int inverse) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total_vec; t += stride) {
        const int64_t vi = t % vec_per_row;
        const int64_t row = t / vec_per_row;
        const int64_t pos = row % rows_per_head;
        const int64_t bh = row / rows_per_head;
        const int64_t b = bh / heads, h = bh % heads;
        const int64_t tok = perm[pos];
        const int64_t src = inverse ? pos : tok;
        const int64_t dst = inverse ? tok : pos;
        const V x = *(const V*)(in + b * in_sb + h * in_sh + src * in_sn + vi * (int64_t)sizeof(V));
        *(V*)(out + b * out_sb + h * out_sh + dst * out_sn + vi * (int64_t)sizeof(V)) = x;
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
    const int64_t total = B * H * N * vec_per_row;
    if (total == 0) return 0;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 workgroups per CU
    if (wide)
        hipLaunchKernelGGL(permute_rows<uint4>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char*)in, (char*)out, N, H, vec_per_row, total, in_sb, in_sh,
                           in_sn, out_sb, out_sh, out_sn, perm, inverse);
    else
        hipLaunchKernelGGL(permute_rows<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const char*)in, (char*)out, N, H, vec_per_row, total, in_sb, in_sh,
                           in_sn, out_sb, out_sh, out_sn, perm, inverse);
    return (int)hipGetLastError();
}
