// The partner branch of pi-Attention's separate-softmax variant
// ("pi-Attention: Online Efficient Sparse Transformers for Long-Context
// Modeling", Section 3.5, Eq. 15): besides the softmax over its local window
// (computed by the attention kernel), every query takes a softmax over its
// online partners N_pi(i) = {x - pi} (and x + pi when both directions are
// fetched; Eq. 9), and the weighted average of their values is added to the
// output (Eq. 11 with the weights of Eq. 15).
//
// This kernel serves the fp32 kernels and the 48-query bf16 kernel (q_block
// 192); the bf16 kernels with 32 queries per wave take the same branch in
// their epilogue.
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

// ---------------------------------------------------------------------------
// Gradients of the separate-softmax variant (bf16).  The two branches are
// independent softmaxes whose outputs add, so their gradients add: the
// window branch's come from the ordinary gradient kernels, given the window
// branch's own row sums delta_i = dout_i . (out_i - partner output_i)
// (pi_skip_bwd_delta), and the partner branch's are added afterwards
// (pi_skip_bwd_grads): for query i with partners p, weights gamma_p =
// softmax_p(z_ip), u_p = dout_i . v_p and dS_p = gamma_p (u_p - sum gamma u),
//     dq_i += scale sum_p dS_p k_p,  dk_p += scale dS_p q_i,  dv_p += gamma_p dout_i.
// A key is the partner of at most two queries (x + pi, and x - pi when both
// directions are fetched), so each row's key gradients are gathered without
// atomics.  One group of G lanes per row as in the forward branch; every lane
// takes part in every group reduction.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = G / 2; off >= 1; off /= 2) x += __shfl_xor(x, off, G);
    return x;
}

template <int D>
struct SkipRow {
    static constexpr int EPL = 8;   // bf16 elements per lane (16 bytes)
    static constexpr int G = D / EPL;
    const NaBwdParams& p;
    int64_t b, h, N;
    int g;
    __device__ int64_t tok(int64_t pos) const { return p.perm ? p.perm[pos] : pos; }
    __device__ void load(const void* base, int64_t sb, int64_t sh, int64_t sn, int64_t t, float* dst) const {
        Elem<uint16_t>::load((const uint16_t*)base + b * sb + h * sh + t * sn + g * EPL, dst);
    }
    // partners of sequence position x: [x - skip, x + skip], -1 = absent
    __device__ void partners(int64_t x, bool valid, int64_t* pt) const {
        pt[0] = valid && x - p.skip >= 0 ? x - p.skip : -1;
        pt[1] = valid && p.skip_both && x + p.skip < N ? x + p.skip : -1;
    }
    // dots of q_i with the partners' keys (times scale) and of dout_i with
    // their values; every lane reduces, absent partners contribute zero
    __device__ void scores(const float* qi, const float* gi, const int64_t* pt, float* z, float* u,
                           float (*kf)[EPL], float (*vf)[EPL]) const {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float dz = 0.f, du = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) kf[t][e] = vf[t][e] = 0.f;
            if (pt[t] >= 0) {
                const int64_t kt = tok(pt[t]);
                load(p.k, p.k_sb, p.k_sh, p.k_sn, kt, kf[t]);
                load(p.v, p.v_sb, p.v_sh, p.v_sn, kt, vf[t]);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    dz = __builtin_fmaf(qi[e], kf[t][e], dz);
                    du = __builtin_fmaf(gi[e], vf[t][e], du);
                }
            }
            z[t] = group_sum<G>(dz) * p.scale;
            u[t] = group_sum<G>(du);
        }
    }
};

// gamma over the present partners (all zero when there is none)
__device__ __forceinline__ void partner_weights(const int64_t* pt, const float* z, float* w) {
    const float m = fmaxf(pt[0] >= 0 ? z[0] : -__builtin_inff(), pt[1] >= 0 ? z[1] : -__builtin_inff());
    float e0 = pt[0] >= 0 ? expf(z[0] - m) : 0.f, e1 = pt[1] >= 0 ? expf(z[1] - m) : 0.f;
    const float l = e0 + e1;
    w[0] = l > 0.f ? e0 / l : 0.f;
    w[1] = l > 0.f ? e1 / l : 0.f;
}

template <int D>
__global__ __launch_bounds__(256) void pi_skip_bwd_delta(NaBwdParams p) {
    using R = SkipRow<D>;
    constexpr int EPL = R::EPL, G = R::G, RPB = 256 / G;
    const int tid = threadIdx.x;
    const int64_t N = p.n_tokens;
    const int64_t total = (int64_t)p.batch * p.heads * N;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const bool valid = row < total;
    const int64_t r = valid ? row : 0;
    const int64_t x = r % N, bh = r / N;
    const R rw{p, bh / p.heads, bh % p.heads, N, tid % G};
    const int64_t xt = rw.tok(x);
    int64_t pt[2];
    rw.partners(x, valid, pt);
    float qi[EPL], gi[EPL], oi[EPL], kf[2][EPL], vf[2][EPL], z[2], u[2], w[2];
    rw.load(p.q, p.q_sb, p.q_sh, p.q_sn, xt, qi);
    rw.load(p.dout, p.g_sb, p.g_sh, p.g_sn, xt, gi);
    rw.load(p.out, p.o_sb, p.o_sh, p.o_sn, xt, oi);
    rw.scores(qi, gi, pt, z, u, kf, vf);
    partner_weights(pt, z, w);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float local = oi[e] - w[0] * vf[0][e] - w[1] * vf[1][e];  // the window branch's output
        d = __builtin_fmaf(gi[e], local, d);
    }
    d = group_sum<G>(d);
    if (valid && rw.g == 0) p.delta[bh * N + xt] = d;
}

template <int D>
__global__ __launch_bounds__(256) void pi_skip_bwd_grads(NaBwdParams p) {
    using R = SkipRow<D>;
    constexpr int EPL = R::EPL, G = R::G, RPB = 256 / G;
    const int tid = threadIdx.x;
    const int64_t N = p.n_tokens;
    const int64_t total = (int64_t)p.batch * p.heads * N;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / G;
    const bool valid = row < total;
    const int64_t r = valid ? row : 0;
    const int64_t x = r % N, bh = r / N;
    const R rw{p, bh / p.heads, bh % p.heads, N, tid % G};
    const int64_t xt = rw.tok(x);
    float kf[2][EPL], vf[2][EPL], z[2], u[2], w[2];

    // ---- x as a query: dq_x += scale sum_p dS_p k_p -------------------------
    {
        int64_t pt[2];
        rw.partners(x, valid, pt);
        float qi[EPL], gi[EPL];
        rw.load(p.q, p.q_sb, p.q_sh, p.q_sn, xt, qi);
        rw.load(p.dout, p.g_sb, p.g_sh, p.g_sn, xt, gi);
        rw.scores(qi, gi, pt, z, u, kf, vf);
        partner_weights(pt, z, w);
        const float ubar = w[0] * u[0] + w[1] * u[1];
        const float ds0 = w[0] * (u[0] - ubar), ds1 = w[1] * (u[1] - ubar);
        if (pt[0] >= 0 || pt[1] >= 0) {
            float acc[EPL];
            uint16_t* dqrow = (uint16_t*)p.dq + rw.b * p.dq_sb + rw.h * p.dq_sh + xt * p.dq_sn + rw.g * EPL;
            Elem<uint16_t>::load(dqrow, acc);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[e] += p.scale * (ds0 * kf[0][e] + ds1 * kf[1][e]);
            Elem<uint16_t>::store(dqrow, acc);
        }
    }
    // ---- x as a key: the queries whose partner it is -------------------------
    float dk[EPL], dv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) dk[e] = dv[e] = 0.f;
    bool any = false;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        // query i = x + skip has partner i - skip = x; query x - skip (both
        // directions) has partner (x - skip) + skip = x
        const int64_t i = c == 0 ? x + p.skip : x - p.skip;
        const bool iv = valid && (c == 0 ? i < N : (p.skip_both && i >= 0));
        const int64_t it = rw.tok(iv ? i : 0);
        int64_t pt[2];
        rw.partners(iv ? i : 0, iv, pt);
        float qi[EPL], gi[EPL];
        rw.load(p.q, p.q_sb, p.q_sh, p.q_sn, it, qi);
        rw.load(p.dout, p.g_sb, p.g_sh, p.g_sn, it, gi);
        rw.scores(qi, gi, pt, z, u, kf, vf);
        partner_weights(pt, z, w);
        const float ubar = w[0] * u[0] + w[1] * u[1];
        // which of i's partners is x: slot 0 (i - skip) for c == 0, slot 1 for c == 1
        const float wx = c == 0 ? w[0] : w[1];
        const float ux = c == 0 ? u[0] : u[1];
        const float ds = wx * (ux - ubar);
        if (iv) {
            any = true;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                dk[e] += p.scale * ds * qi[e];
                dv[e] += wx * gi[e];
            }
        }
    }
    if (any) {
        float acc[EPL];
        uint16_t* dkrow = (uint16_t*)p.dk + rw.b * p.dk_sb + rw.h * p.dk_sh + xt * p.dk_sn + rw.g * EPL;
        Elem<uint16_t>::load(dkrow, acc);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += dk[e];
        Elem<uint16_t>::store(dkrow, acc);
        uint16_t* dvrow = (uint16_t*)p.dv + rw.b * p.dv_sb + rw.h * p.dv_sh + xt * p.dv_sn + rw.g * EPL;
        Elem<uint16_t>::load(dvrow, acc);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += dv[e];
        Elem<uint16_t>::store(dvrow, acc);
    }
}

template <int D, bool GRADS>
int launch_skip_bwd(const NaBwdParams& p, hipStream_t st) {
    constexpr int RPB = 256 / SkipRow<D>::G;
    const int64_t total = (int64_t)p.batch * p.heads * p.n_tokens;
    const int64_t blocks = (total + RPB - 1) / RPB;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    if (GRADS)
        hipLaunchKernelGGL((pi_skip_bwd_grads<D>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((pi_skip_bwd_delta<D>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

int na_skip_bwd_delta_launch(const NaBwdParams& p, int head_dim, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (head_dim == 64) return launch_skip_bwd<64, false>(p, st);
    if (head_dim == 128) return launch_skip_bwd<128, false>(p, st);
    return (int)hipErrorInvalidValue;
}

int na_skip_bwd_grads_launch(const NaBwdParams& p, int head_dim, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (head_dim == 64) return launch_skip_bwd<64, true>(p, st);
    if (head_dim == 128) return launch_skip_bwd<128, true>(p, st);
    return (int)hipErrorInvalidValue;
}

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
