// Fused block-sparse local-attention forward for gfx950 (MI355X).
//
// One workgroup owns one query tile of one (batch, head) and walks only the
// non-empty key/value tiles of that query tile (the plan's CSR row).  For each
// key/value tile it stages K and V in LDS, computes the transposed score block
// S^T = K Q^T with MFMA (so that each lane owns one query and the row maximum
// needs a single cross-lane step), applies the per-element window mask only
// when the tile is partial (or runs past the last token), updates an fp32
// online softmax in the log2 domain and accumulates O^T = V^T P^T with MFMA.
// The epilogue divides by the row sum and writes O and the natural-log LSE.
//
// Mathematics: softmax attention restricted to a key set ("pi-Attention",
// Eqs. 2-4 with the sum of Eq. 3 over the neighbourhood), evaluated tile by
// tile with on-chip accumulation (same page, "Hardware-aware online
// execution"); tiles classified empty / partial / full ("Hilbert-Guided Sparse
// Local Attention", methodology).
//
// MFMA 32x32 accumulator layout used throughout: lane l, element r holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32.  A and B operands: lane l holds
// row (A) / column (B) l%32 and reduction slots 8*(l/32)..8*(l/32)+7 (bf16) or
// slot l/32 (fp32).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "na_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (NaN preserved).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
    u32x4 w;
    w[0] = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
    w[1] = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
    w[2] = bf16_bits(v[4]) | (bf16_bits(v[5]) << 16);
    w[3] = bf16_bits(v[6]) | (bf16_bits(v[7]) << 16);
    return __builtin_bit_cast(bf16x8, w);
}

// Window test of one key (pattern coordinates kc) against a query box
// (lo[3], hi[3]); dilation: the key must sit on the query's sub-grid.
__device__ __forceinline__ bool in_window(const int32_t* lo, const int32_t* hi, int4 kc,
                                          const NaAttnParams& p) {
    bool ok = kc.x >= lo[0] && kc.x < hi[0];
    if (p.pdims > 1) ok = ok && kc.y >= lo[1] && kc.y < hi[1];
    if (p.pdims > 2) ok = ok && kc.z >= lo[2] && kc.z < hi[2];
    if (p.has_dilation) {
        ok = ok && (kc.x - lo[0]) % p.dil0 == 0;
        if (p.pdims > 1) ok = ok && (kc.y - lo[1]) % p.dil1 == 0;
        if (p.pdims > 2) ok = ok && (kc.z - lo[2]) % p.dil2 == 0;
    }
    return ok;
}

// ---------------------------------------------------------------------------
// bf16: NW waves, 32 queries per wave (query tile 32*NW), key/value tile 64.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16(NaAttnParams p) {
    constexpr int KV = NA_KV_BLOCK_BF16;
    constexpr int NT = NW * 64;
    constexpr int QB = 32 * NW;
    constexpr int ROW = D + 8;                 // LDS row stride (elements): 16 B pad
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int CH = KV * CPR / NT;          // chunks per thread per tensor
    static_assert(KV * CPR % NT == 0, "tile does not split evenly");
    constexpr int KS = D / 16;                 // QK reduction steps
    constexpr int DB = D / 32;                 // PV output blocks

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[KV * ROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[KV * ROW];
    __shared__ int4 kc_lds[KV];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    const int wg = blockIdx.x;
    const int qt = wg % p.n_q_tiles;
    const int bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;

    // ---- this lane's query -------------------------------------------------
    const int qpos = qt * QB + wave * 32 + l32;
    const bool qvalid = qpos < N;
    const int qtok = qvalid ? (p.perm ? p.perm[qpos] : qpos) : 0;
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qtok * p.q_sn;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qvalid) w = *(const u32x4*)(qrow + 16 * s + 8 * half);
            qf[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
    int32_t qlo[3] = {0, 0, 0}, qhi[3] = {0, 0, 0};
    if (p.qbox && qvalid) {
        const int4 a = *(const int4*)(p.qbox + (int64_t)qpos * 8);
        const int4 c = *(const int4*)(p.qbox + (int64_t)qpos * 8 + 4);
        qlo[0] = a.x; qlo[1] = a.y; qlo[2] = a.z;
        qhi[0] = a.w; qhi[1] = c.x; qhi[2] = c.y;
    }

    const uint16_t* kbase = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh;
    const uint16_t* vbase = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh;

    // ---- register staging of one key/value tile ----------------------------
    u32x4 kreg[CH], vreg[CH];
    int4 kcreg = {0, 0, 0, 0};
    auto load_tile = [&](uint32_t entry) {
        const int kt = (int)(entry & ~NA_ENTRY_PARTIAL);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            const int row = c / CPR, col = (c % CPR) * 8;
            const int kp = kt * KV + row;
            u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
            if (kp < N) {
                const int tok = p.perm ? p.perm[kp] : kp;
                kw = *(const u32x4*)(kbase + (int64_t)tok * p.k_sn + col);
                vw = *(const u32x4*)(vbase + (int64_t)tok * p.v_sn + col);
            }
            kreg[i] = kw;
            vreg[i] = vw;
        }
        if ((entry & NA_ENTRY_PARTIAL) && tid < KV) {
            const int kp = kt * KV + tid;
            kcreg = kp < N ? *(const int4*)(p.kcoord + (int64_t)kp * 4) : int4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](uint32_t entry) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + NT * i;
            const int row = c / CPR, col = (c % CPR) * 8;
            *(u32x4*)(k_lds + row * ROW + col) = kreg[i];
            *(u32x4*)(v_lds + row * ROW + col) = vreg[i];
        }
        if ((entry & NA_ENTRY_PARTIAL) && tid < KV) kc_lds[tid] = kcreg;
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    const int e0 = p.row_ptr[qt], e1 = p.row_ptr[qt + 1];
    if (e0 < e1) load_tile(p.entries[e0]);
    for (int e = e0; e < e1; ++e) {
        const uint32_t entry = p.entries[e];
        store_tile(entry);
        __syncthreads();
        if (e + 1 < e1) load_tile(p.entries[e + 1]);

        const int kt = (int)(entry & ~NA_ENTRY_PARTIAL);
        // S^T = K Q^T for the two 32-key halves of the tile.
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *(const bf16x8*)(k_lds + (32 * kb + l32) * ROW + 16 * ks + 8 * half);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
            }
        }
        // scale into the log2 domain; mask if partial or ragged
        const bool partial = (entry & NA_ENTRY_PARTIAL) != 0;
        const bool ragged = kt * KV + KV > N;
        float mt = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kb][r] * p.scale_log2;
                if (partial || ragged) {
                    const int key = 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                    bool ok = kt * KV + key < N;
                    if (partial && ok) ok = in_window(qlo, qhi, kc_lds[key], p);
                    x = ok ? x : kNegInf;
                }
                s[kb][r] = x;
                mt = fmaxf(mt, x);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pe = fast_exp2(s[kb][r] - m_use);
                s[kb][r] = pe;
                l_run += pe;
            }
        // O^T += V^T P^T, 16 keys per step: P^T slot j of half h is the score
        // of key 16*ks + 8*(j/4) + 4*h + j%4, i.e. accumulator elements
        // 8*(ks%2)..+7 of block ks/2.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = s[ks / 2][8 * (ks % 2) + j];
            const bf16x8 bp = pack8(pv);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 32 * db + l32;
                uint16_t va[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int key = 16 * ks + 8 * (j / 4) + 4 * half + (j % 4);
                    va[j] = v_lds[key * ROW + d];
                }
                u32x4 w;
                w[0] = va[0] | ((uint32_t)va[1] << 16);
                w[1] = va[2] | ((uint32_t)va[3] << 16);
                w[2] = va[4] | ((uint32_t)va[5] << 16);
                w[3] = va[6] | ((uint32_t)va[7] << 16);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), bp,
                                                                o[db], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue -----------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!qvalid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = (uint16_t*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)qtok * p.o_sn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * half;
            u16x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (uint16_t)bf16_bits(o[db][4 * g + i] * inv);
            *(u16x4*)(orow + d) = w;
        }
    if (p.lse && half == 0) {
        const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        p.lse[(int64_t)bh * N + qtok] = lse;
    }
}

// ---------------------------------------------------------------------------
// fp32: one wave, 32 queries, key/value tile 32, fp32 MFMA (no bf16 anywhere).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32(NaAttnParams p) {
    constexpr int KV = NA_KV_BLOCK_F32;
    constexpr int ROW = D + 1;      // odd stride: conflict-free column reads
    constexpr int KS = D / 2;
    constexpr int DB = D / 32;
    __shared__ float k_lds[KV * ROW];
    __shared__ float v_lds[KV * ROW];
    __shared__ int4 kc_lds[KV];

    const int lane = threadIdx.x;
    const int half = lane >> 5, l32 = lane & 31;
    const int wg = blockIdx.x;
    const int qt = wg % p.n_q_tiles;
    const int bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;

    const int qpos = qt * 32 + l32;
    const bool qvalid = qpos < N;
    const int qtok = qvalid ? (p.perm ? p.perm[qpos] : qpos) : 0;
    float qf[KS];
    {
        const float* qrow = (const float*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qtok * p.q_sn;
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[s] = qvalid ? qrow[2 * s + half] : 0.f;
    }
    int32_t qlo[3] = {0, 0, 0}, qhi[3] = {0, 0, 0};
    if (p.qbox && qvalid) {
        const int32_t* bx = p.qbox + (int64_t)qpos * 8;
        for (int i = 0; i < 3; ++i) {
            qlo[i] = bx[i];
            qhi[i] = bx[3 + i];
        }
    }
    const float* kbase = (const float*)p.k + b * p.k_sb + h * p.k_sh;
    const float* vbase = (const float*)p.v + b * p.v_sb + h * p.v_sh;

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    const int e0 = p.row_ptr[qt], e1 = p.row_ptr[qt + 1];
    for (int e = e0; e < e1; ++e) {
        const uint32_t entry = p.entries[e];
        const int kt = (int)(entry & ~NA_ENTRY_PARTIAL);
        const bool partial = (entry & NA_ENTRY_PARTIAL) != 0;
        // stage the tile: lane handles key rows lane%32, half of the columns each
        for (int row = 0; row < KV; ++row) {
            const int kp = kt * KV + row;
            const int tok = kp < N ? (p.perm ? p.perm[kp] : kp) : -1;
            for (int c = lane; c < D; c += 64) {
                k_lds[row * ROW + c] = tok >= 0 ? kbase[(int64_t)tok * p.k_sn + c] : 0.f;
                v_lds[row * ROW + c] = tok >= 0 ? vbase[(int64_t)tok * p.v_sn + c] : 0.f;
            }
        }
        if (partial && lane < KV) {
            const int kp = kt * KV + lane;
            kc_lds[lane] = kp < N ? *(const int4*)(p.kcoord + (int64_t)kp * 4) : int4{0, 0, 0, 0};
        }
        __syncthreads();

        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k_lds[l32 * ROW + 2 * ks + half], qf[ks], s, 0,
                                                     0, 0);
        const bool ragged = kt * KV + KV > N;
        float mt = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = s[r] * p.scale_log2;
            if (partial || ragged) {
                const int key = 8 * (r / 4) + 4 * half + (r % 4);
                bool ok = kt * KV + key < N;
                if (partial && ok) ok = in_window(qlo, qhi, kc_lds[key], p);
                x = ok ? x : kNegInf;
            }
            s[r] = x;
            mt = fmaxf(mt, x);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = fast_exp2(s[r] - m_use);
            l_run += s[r];
        }
        // O^T += V^T P^T, one key per step: element r of this lane is key
        // 8*(r/4) + 4*half + r%4, which is the reduction slot `half` of step r.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r / 4) + 4 * half + (r % 4);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(v_lds[key * ROW + 32 * db + l32], s[r],
                                                             o[db], 0, 0, 0);
        }
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!qvalid) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = (float*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)qtok * p.o_sn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * half;
            float4 w = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                        o[db][4 * g + 3] * inv};
            *(float4*)(orow + d) = w;
        }
    if (p.lse && half == 0) {
        const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        p.lse[(int64_t)bh * N + qtok] = lse;
    }
}

}  // namespace

bool na_attn_supported(int dtype, int head_dim, int q_block, int kv_block) {
    if (dtype == NA_BF16)
        return (head_dim == 64 || head_dim == 128) && kv_block == NA_KV_BLOCK_BF16 &&
               (q_block == 128 || q_block == 256);
    if (dtype == NA_F32)
        return (head_dim == 32 || head_dim == 64) && kv_block == NA_KV_BLOCK_F32 &&
               q_block == NA_Q_BLOCK_F32;
    return false;
}

int na_attn_launch(const NaAttnParams& p, int dtype, int head_dim, int q_block, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const dim3 grid((unsigned)p.n_wg);
    if (dtype == NA_BF16) {
        if (head_dim == 128 && q_block == 128)
            hipLaunchKernelGGL((attn_fwd_bf16<128, 4>), grid, dim3(256), 0, st, p);
        else if (head_dim == 128 && q_block == 256)
            hipLaunchKernelGGL((attn_fwd_bf16<128, 8>), grid, dim3(512), 0, st, p);
        else if (head_dim == 64 && q_block == 128)
            hipLaunchKernelGGL((attn_fwd_bf16<64, 4>), grid, dim3(256), 0, st, p);
        else if (head_dim == 64 && q_block == 256)
            hipLaunchKernelGGL((attn_fwd_bf16<64, 8>), grid, dim3(512), 0, st, p);
        else
            return (int)hipErrorInvalidValue;
    } else {
        if (head_dim == 32)
            hipLaunchKernelGGL((attn_fwd_f32<32>), grid, dim3(64), 0, st, p);
        else if (head_dim == 64)
            hipLaunchKernelGGL((attn_fwd_f32<64>), grid, dim3(64), 0, st, p);
        else
            return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}
