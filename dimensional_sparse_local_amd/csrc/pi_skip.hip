// The partner branch of pi-Attention's separate-softmax variant
// ("pi-Attention: Online Efficient Sparse Transformers for Long-Context
// Modeling", Section 3.5, Eq. 15): besides the softmax over its local window
// (computed by the attention kernel), every query takes a softmax over its
// online partners N_pi(i) = {x - pi} (and x + pi when both directions are
// fetched; Eq. 9), and the weighted average of their values is added to the
// output (Eq. 11 with the weights of Eq. 15).
//
// One group of G lanes per query row, 16 bytes of each row per lane: the group
// reduces its partial dot products by shuffles, takes the (at most 2-way)
// softmax and accumulates the partners' value rows into the output row, which
// the attention kernel wrote before on the same stream.  Memory bound: a query
// reads its q row, at most two key and value rows and its output row.
#include <hip/hip_runtime.h>

#include "attn_common.h"

namespace {

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {  // bf16 bits
    static constexpr int kPerLane = 8;
    static __device__ void load(const uint16_t* src, float* dst) {
        const u32x4 w = *(const u32x4*)src;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            dst[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    }
    static __device__ void store(uint16_t* dst, const float* src) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2 x = {src[2 * i], src[2 * i + 1]};
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
        }
        *(u32x4*)dst = w;
    }
};
template <> struct Elem<float> {
    static constexpr int kPerLane = 4;
    static __device__ void load(const float* src, float* dst) {
        const f32x4 w = *(const f32x4*)src;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = w[i];
    }
    static __device__ void store(float* dst, const float* src) {
        *(f32x4*)dst = f32x4{src[0], src[1], src[2], src[3]};
    }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void pi_skip_branch(NaSkipParams p) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int G = D / EPL;        // lanes per query row: 8 or 16
    constexpr int RPB = 256 / G;      // rows per block
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "row group must divide a wave");
    const int tid = threadIdx.x;
    const int g = tid % G;
    const int64_t N = p.n_tokens;
    const int64_t total = (int64_t)p.batch * p.heads * N;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const bool valid = row < total;   // uniform inside a group
    const int64_t r = valid ? row : 0;
    const int64_t x = r % N;          // sequence position = pattern coordinate
    const int64_t bh = r / N;
    const int64_t b = bh / p.heads, h = bh % p.heads;
    const int64_t qtok = p.perm ? p.perm[x] : x;

    // partners, as sequence positions; -1 = absent
    int64_t part[2];
    part[0] = x - p.skip >= 0 ? x - p.skip : -1;
    part[1] = p.skip_both && x + p.skip < N ? x + p.skip : -1;
    if (!valid) part[0] = part[1] = -1;

    float qf[EPL];
    Elem<T>::load((const T*)p.q + b * p.q_sb + h * p.q_sh + qtok * p.q_sn + g * EPL, qf);
    float z[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float dot = 0.f;
        if (part[t] >= 0) {
            const int64_t tok = p.perm ? p.perm[part[t]] : part[t];
            float kf[EPL];
            Elem<T>::load((const T*)p.k + b * p.k_sb + h * p.k_sh + tok * p.k_sn + g * EPL, kf);
#pragma unroll
            for (int i = 0; i < EPL; ++i) dot = __builtin_fmaf(qf[i], kf[i], dot);
        }
        // every lane of the group takes part in the reduction
#pragma unroll
        for (int off = G / 2; off >= 1; off /= 2) dot += __shfl_xor(dot, off, G);
        z[t] = dot * p.scale;
    }
    if (part[0] < 0 && part[1] < 0) return;  // no partner: the branch adds nothing
    const float m = fmaxf(part[0] >= 0 ? z[0] : -__builtin_inff(),
                          part[1] >= 0 ? z[1] : -__builtin_inff());
    float e[2], l = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        e[t] = part[t] >= 0 ? expf(z[t] - m) : 0.f;
        l += e[t];
    }
    float acc[EPL];
    T* orow = (T*)p.out + b * p.o_sb + h * p.o_sh + qtok * p.o_sn + g * EPL;
    Elem<T>::load(orow, acc);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (part[t] < 0) continue;
        const int64_t tok = p.perm ? p.perm[part[t]] : part[t];
        float vf[EPL];
        Elem<T>::load((const T*)p.v + b * p.v_sb + h * p.v_sh + tok * p.v_sn + g * EPL, vf);
        const float w = e[t] / l;
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] = __builtin_fmaf(w, vf[i], acc[i]);
    }
    Elem<T>::store(orow, acc);
}

template <typename T, int D>
int launch(const NaSkipParams& p, hipStream_t st) {
    constexpr int RPB = 256 / (D / Elem<T>::kPerLane);
    const int64_t total = (int64_t)p.batch * p.heads * p.n_tokens;
    const int64_t blocks = (total + RPB - 1) / RPB;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((pi_skip_branch<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

bool na_skip_supported(int dtype, int head_dim) {
    if (dtype == NA_BF16) return head_dim == 64 || head_dim == 128;
    if (dtype == NA_F32) return head_dim == 32 || head_dim == 64;
    return false;
}

int na_skip_launch(const NaSkipParams& p, int dtype, int head_dim, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (dtype == NA_BF16 && head_dim == 64) return launch<uint16_t, 64>(p, st);
    if (dtype == NA_BF16 && head_dim == 128) return launch<uint16_t, 128>(p, st);
    if (dtype == NA_F32 && head_dim == 32) return launch<float, 32>(p, st);
    if (dtype == NA_F32 && head_dim == 64) return launch<float, 64>(p, st);
    return (int)hipErrorInvalidValue;
}
