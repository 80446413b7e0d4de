// Gradients of the fused block-sparse local attention for gfx950 (MI355X).
//
// With P_ij = exp(scale q_i . k_j - lse_i) over the neighbourhood of query i,
// the gradients of sum_i dout_i . out_i are ("pi-Attention", gradient analysis
// of adaptive fusion, Eq. 23: the softmax Jacobian)
//     dP_ij = dout_i . v_j,   dS_ij = P_ij (dP_ij - delta_i),
//     delta_i = sum_j P_ij dP_ij = dout_i . out_i,
//     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//     dv_j = sum_i P_ij dout_i.
// Three kernels:
//   bwd_delta      delta_i from dout and the forward's out (fp32),
//   attn_bwd_dq    query-major: the forward's walk over each query tile's
//                  non-empty key tiles, recomputing S and dP, accumulating dq,
//   attn_bwd_dkdv  key-major: each key tile walks the query tiles that attend
//                  it (the plan's transposed map) in steps of 32 queries,
//                  accumulating dk and dv.
// Every pair (q_i, k_j) is visited exactly where the forward visited it, with
// the same tile classes and masks; P is recomputed from the stored lse, so no
// running maximum is needed.  P and dS are rounded to bf16 for their MFMA
// products; accumulation is fp32.
#include "attn_common.h"

#include <mutex>

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// lse in the log2 domain; a query with an empty neighbourhood (lse = -inf) or
// past the last token gets +inf, which makes every P of its row exactly 0.
__device__ __forceinline__ float lse_log2(float lse, bool valid) {
    constexpr float kLog2e = 1.4426950408889634f;
    return valid && lse > kNegInf ? lse * kLog2e : __builtin_inff();
}

// Store a 32 (rows d) x 32 (columns = this lane's token) block set in the
// accumulator layout, times f, as bf16 into row `row` of a [N, D] slice.
template <int DB>
__device__ __forceinline__ void store_rows_t(uint16_t* row, const f32x16* acc, float f, int half) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * half;
            const f32x2 x0 = {acc[db][4 * g] * f, acc[db][4 * g + 1] * f};
            const f32x2 x1 = {acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f};
            const uint2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(x0, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(x1, bf16x2))};
            *(uint2*)(row + d) = w;
        }
}

// ---------------------------------------------------------------------------
// delta_i = dout_i . out_i (fp32 sum of bf16 products), row-major token order.
// D / 8 lanes per row, 8 elements each.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta(NaBwdParams p) {
    constexpr int L = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / L;
    const int sub = (int)(gid % L);
    const int64_t total = (int64_t)p.batch * p.heads * p.n_tokens;
    float acc = 0.f;
    if (row < total) {
        const int64_t bh = row / p.n_tokens, n = row % p.n_tokens;
        const int64_t b = bh / p.heads, h = bh % p.heads;
        const u32x4 o = *(const u32x4*)((const uint16_t*)p.out + b * p.o_sb + h * p.o_sh + n * p.o_sn +
                                        8 * sub);
        const u32x4 g = *(const u32x4*)((const uint16_t*)p.dout + b * p.g_sb + h * p.g_sh +
                                        n * p.g_sn + 8 * sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < total && sub == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dq: NW waves of 32 queries (query tile 32 * NW), key/value tile 64, the
// forward's walk and staging (attn_fwd_bf16): K and V tiles by LDS DMA into
// two statically selected buffers, the next tile in flight while one is
// computed.  Per key tile, with S^T and dP^T in the accumulator layout of the
// forward (lane = query, K rows permuted inside the MFMA block):
//     S^T  = K Q^T,  dP^T = V dout^T       (K and V rows as A operands),
//     P^T  = exp2(S^T scale log2 e - lse log2 e),  dS^T = P^T (dP^T - delta),
//     dq^T += K^T dS^T                      (K^T by transposing LDS reads).
// ---------------------------------------------------------------------------
template <int D, int NW, bool BIAS = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq(NaBwdParams p) {
    using MaskT = typename MaskRow<BIAS>::T;
    constexpr int KV = NA_KV_BLOCK_BF16;
    constexpr int QB = 32 * NW;
    constexpr int ROW = D + 8;
    constexpr int CS = D / 8 + 1;
    constexpr int TILE = KV * ROW;
    constexpr int NI = CS;
    constexpr int IPW = (NI + NW - 1) / NW;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;

    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    const int n_wg = p.n_q_tiles * p.batch * p.heads;
    const int wg = xcd_remap(blockIdx.x, n_wg);
    const int qt = wg % p.n_q_tiles;
    const int bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;
    const float c = p.scale_log2;

    // ---- this lane's query -------------------------------------------------
    const int qpos = qt * QB + wave * 32 + l32;
    const bool qvalid = qpos < N;
    const int qtok = qvalid ? (p.perm ? p.perm[qpos] : qpos) : 0;
    bf16x8 qf[KS], gf[KS];
    {
        const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qtok * p.q_sn;
        const uint16_t* grow =
            (const uint16_t*)p.dout + b * p.g_sb + h * p.g_sh + (int64_t)qtok * p.g_sn;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 w = {0u, 0u, 0u, 0u}, x = {0u, 0u, 0u, 0u};
            if (qvalid) {
                w = *(const u32x4*)(qrow + 16 * s + 8 * half);
                x = *(const u32x4*)(grow + 16 * s + 8 * half);
            }
            qf[s] = __builtin_bit_cast(bf16x8, w);
            gf[s] = __builtin_bit_cast(bf16x8, x);
        }
    }
    // fixed fusion: the forward's lse carries log(alpha) (every logit's common
    // prior); without it the window keys need no bias and the partners p.skip_bias
    const float lse_raw = qvalid ? p.lse[(int64_t)bh * N + qtok] : 0.f;
    const float neg_lse2 = -lse_log2(BIAS ? lse_raw - p.lse_shift : lse_raw, qvalid);
    const float dlt = qvalid ? p.delta[(int64_t)bh * N + qtok] : 0.f;
    const uint16_t* kbase = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh;
    const uint16_t* vbase = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh;
    const int mrow = wave * 32 + l32;

    // DMA of a key/value tile, as in the forward: block j = wave + NW*i moves
    // slots 64*j .. 64*j+63, slot = (row, chunk), the pad chunk re-reads chunk 0
    int dma_row[IPW], dma_off[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int slot = 64 * (wave + NW * i) + lane;
        dma_row[i] = slot / CS;
        const int ch = slot % CS;
        dma_off[i] = ch < CS - 1 ? 8 * ch : 0;
    }
    auto tokens = [&](NaEntry entry, int* tok) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int kp = min(entry.kt * KV + dma_row[i], N - 1);
            tok[i] = p.perm ? gload(p.perm + kp) : kp;
        }
    };
    auto issue = [&](NaEntry entry, const int* tok, uint16_t* kl, uint16_t* vl) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int blk = wave + NW * i;
            if (blk < NI) {
                const bool real = entry.kt * KV + dma_row[i] < N;
                const uint16_t* gk = real ? kbase + ((uint32_t)tok[i] * (uint32_t)p.k_sn + dma_off[i])
                                          : (const uint16_t*)p.zero;
                const uint16_t* gv = real ? vbase + ((uint32_t)tok[i] * (uint32_t)p.v_sn + dma_off[i])
                                          : (const uint16_t*)p.zero;
                dma16(gk, kl + blk * 512);
                dma16(gv, vl + blk * 512);
            }
        }
    };
    // The mask row is loaded unconditionally (the zero page stands in for a
    // tile without a mask, whose words are never read): a load merged with a
    // constant would be consumed at once, and that wait would also cover the
    // K/V rows just sent to LDS.
    auto mask_row = [&](NaEntry entry) {
        MaskT w;
        const int64_t at = ((int64_t)entry.mask * QB + mrow) * 2;
        const bool has = entry.mask >= 0;
        const u32x2 keep = gload((const u32x2*)(has ? p.masks + at : (const uint32_t*)p.zero));
        w[0] = keep[0];
        w[1] = keep[1];
        if constexpr (BIAS) {
            const u32x2 part = gload((const u32x2*)(has ? p.skip_masks + at : (const uint32_t*)p.zero));
            w[2] = part[0];
            w[3] = part[1];
        }
        return w;
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // K rows inside a 32-key MFMA block are permuted as in the forward, so the
    // accumulator elements of S^T / dP^T are the B-operand slots of dS^T.
    const int kappa = 16 * (l32 >> 4) + 2 * ((l32 >> 3) & 1) + ((l32 >> 2) & 1) + 4 * (l32 & 3);
    const int tr_base = (half + 4 * ((lane & 15) >> 2)) * ROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    auto compute = [&](NaEntry entry, MaskT mk, const uint16_t* kl, const uint16_t* vl) {
        f32x16 s[2], dp[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = dp[0][r] = dp[1][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint16_t* kr = kl + (kappa + 32 * kb) * ROW + 8 * half;
            const uint16_t* vr = vl + (kappa + 32 * kb) * ROW + 8 * half;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kr + 16 * ks), qf[ks],
                                                                s[kb], 0, 0, 0);
                dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vr + 16 * ks), gf[ks],
                                                                 dp[kb], 0, 0, 0);
            }
        }
        // element mask: score (kb, r) is key 32*kb + 16*(r/8) + 2*(r/4 % 2) + half + 4*(r % 4)
        if (entry.mask >= 0) {
            const uint32_t w0 = mk[0] >> half, w1 = mk[1] >> half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int bit = 16 * (r / 8) + 2 * ((r / 4) % 2) + 4 * (r % 4);
                s[0][r] = keep_if(w0, bit, s[0][r]);
                s[1][r] = keep_if(w1, bit, s[1][r]);
            }
            if constexpr (BIAS) {
                const uint32_t b0 = mk[2] >> half, b1 = mk[3] >> half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int bit = 16 * (r / 8) + 2 * ((r / 4) % 2) + 4 * (r % 4);
                    s[0][r] += ((b0 >> bit) & 1u) ? p.skip_bias : 0.f;
                    s[1][r] += ((b1 >> bit) & 1u) ? p.skip_bias : 0.f;
                }
            }
        }
        // P^T and dS^T in place of S^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(s[kb][r], c, neg_lse2));
                s[kb][r] = pr * (dp[kb][r] - dlt);
            }
        // dq^T += K^T dS^T, 16 keys per step (the transposing reads deliver the
        // K rows in the order of the accumulator slots, as V^T in the forward)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f32x16& sv = s[ks / 2];
            const int r0 = 8 * (ks % 2);
            const bf16x8 bd = cvt8(sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3], sv[r0 + 4], sv[r0 + 5],
                                   sv[r0 + 6], sv[r0 + 7]);
            const uint16_t* kr = kl + tr_base + 16 * ks * ROW;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x4 lo = lds_read_tr(kr + 32 * db);
                const bf16x4 hi = lds_read_tr(kr + 2 * ROW + 32 * db);
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bd, acc[db], 0, 0, 0);
            }
        }
    };

    // ---- pipelined walk over the CSR row (as in the forward) -----------------
    const int e0 = cload(p.row_ptr + qt), e1 = cload(p.row_ptr + qt + 1);
    const NaEntry none = {0, -1};
    NaEntry ent_a = none, ent_b = none, ent_c = none;
    int tok_n[IPW];
    MaskT mk_a = {}, mk_b = {};
    if (e0 < e1) {
        ent_a = load_entry(p.entries + e0);
        if (e0 + 1 < e1) ent_b = load_entry(p.entries + e0 + 1);
        if (e0 + 2 < e1) ent_c = load_entry(p.entries + e0 + 2);
        int tok0[IPW];
        tokens(ent_a, tok0);
        issue(ent_a, tok0, k_lds0, v_lds0);
        mk_a = mask_row(ent_a);
        if (e0 + 1 < e1) {
            tokens(ent_b, tok_n);
            mk_b = mask_row(ent_b);
        }
    }
    auto step = [&](int e, const uint16_t* kl, const uint16_t* vl, uint16_t* kn, uint16_t* vn) {
        wait_vmem();
        __syncthreads();
        if (e + 1 < e1) issue(ent_b, tok_n, kn, vn);
        if (e + 2 < e1) tokens(ent_c, tok_n);
        const MaskT mk_c = mask_row(ent_c);   // ent_c is `none` past the row's end
        const NaEntry ent_d = e + 3 < e1 ? load_entry(p.entries + e + 3) : none;
        compute(ent_a, mk_a, kl, vl);
        ent_a = ent_b;
        ent_b = ent_c;
        ent_c = ent_d;
        mk_a = mk_b;
        mk_b = mk_c;
    };
    for (int e = e0; e < e1; e += 2) {
        step(e, k_lds0, v_lds0, k_lds1, v_lds1);
        if (e + 1 < e1) step(e + 1, k_lds1, v_lds1, k_lds0, v_lds0);
    }
    // no DMA may still be writing this workgroup's LDS when it ends
    wait_vmem();
    if (!qvalid) return;
    store_rows_t<DB>((uint16_t*)p.dq + b * p.dq_sb + h * p.dq_sh + (int64_t)qtok * p.dq_sn, acc,
                     p.scale, half);
}

// ---------------------------------------------------------------------------
// dk, dv: one workgroup per pair of key/value tiles (128 keys) of one (batch,
// head), four waves of 32 keys (one per SIMD).  The keys and values stay in
// registers as B operands; the workgroup walks the query tiles that attend
// either tile (the plan's paired key-major map) in steps of 32 queries,
// staging their q and dout rows in LDS by DMA (double-buffered, the next step
// in flight) together with their lse, delta and the mask words of both tiles.
// Staging one step for 128 keys instead of 64 halves the staged bytes per
// flop.  A wave whose tile the step's query tile does not attend skips the
// step's arithmetic.  Per step, with the roles of the forward swapped
// (lane = key, q / dout rows permuted inside the MFMA block):
//     S = Q K^T,  dP = dout V^T               (q and dout rows as A operands),
//     P = exp2(S scale log2 e - lse log2 e),  dS = P (dP - delta),
//     dv^T += dout^T P,  dk^T += Q^T dS       (transposing LDS reads).
// The accumulator element r of half h of S and dP holds query
// 16*(r/8) + 2*(r/4 % 2) + h + 4*(r%4) of the step; lse and delta are staged in
// that order so that each lane reads its sixteen as four 16-byte words.
// ---------------------------------------------------------------------------
template <int D, bool BIAS = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2, 2)))   // two waves per SIMD: <= 256 registers
void attn_bwd_dkdv(NaBwdParams p) {
    constexpr int KV = NA_KV_BLOCK_BF16;
    constexpr int NW = 4;
    constexpr int QS = 32;                       // queries per step
    constexpr int ROW = D + 8;
    constexpr int CS = D / 8 + 1;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int RSLOT = QS * CS;               // 16-byte slots of one tensor's rows
    constexpr int NBLK = 2 * RSLOT / 64;         // 1 KB DMA blocks per step (q and dout)
    static_assert(2 * RSLOT % 64 == 0, "q and dout rows fill whole DMA blocks");
    constexpr int BPW = (NBLK + NW - 1) / NW;
    constexpr int RE = 2 * QS * ROW;             // LDS elements of a step's rows
    // lse (log2), delta, mask words [2][QS][2] (and partner words [2][QS][2])
    constexpr int AUX = 2 * QS + 4 * QS + (BIAS ? 4 * QS : 0);

    __shared__ __attribute__((aligned(1024))) uint16_t rows0[RE];
    __shared__ __attribute__((aligned(1024))) uint16_t rows1[RE];
    __shared__ __attribute__((aligned(16))) float aux0[AUX];
    __shared__ __attribute__((aligned(16))) float aux1[AUX];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    const int n_pairs = (p.n_kv_tiles + 1) / 2;
    const int n_wg = n_pairs * p.batch * p.heads;
    const int wg = xcd_remap(blockIdx.x, n_wg);
    const int kg = wg % n_pairs;              // key tiles 2 kg and 2 kg + 1
    const int bh = wg / n_pairs;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;
    const int QBK = p.q_block;
    const int nsub = QBK / QS;
    const float c = p.scale_log2;

    // ---- this lane's key ------------------------------------------------------
    const int kpos = kg * 2 * KV + 32 * wave + l32;   // waves 0-1: tile 2 kg, 2-3: 2 kg + 1
    const bool kvalid = kpos < N;
    const int ktok = kvalid ? (p.perm ? p.perm[kpos] : kpos) : 0;
    bf16x8 kf[KS];
    // At D = 128 the V fragments wait in LDS (each lane reads back its own
    // 16-byte words, one read per dP MFMA): 32 registers fewer, which lets two
    // waves share a SIMD and hide each other's LDS and softmax latency.  At
    // D = 64 they fit in registers (16) at the same occupancy.
    constexpr bool VREG = D == 64;
    __shared__ __attribute__((aligned(16))) u32x4 vfrag[VREG ? 1 : NW * KS * 64];
    u32x4 vreg[KS];
    {
        const uint16_t* krow = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh + (int64_t)ktok * p.k_sn;
        const uint16_t* vrow = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh + (int64_t)ktok * p.v_sn;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 w = {0u, 0u, 0u, 0u}, x = {0u, 0u, 0u, 0u};
            if (kvalid) {
                w = *(const u32x4*)(krow + 16 * s + 8 * half);
                x = *(const u32x4*)(vrow + 16 * s + 8 * half);
            }
            kf[s] = __builtin_bit_cast(bf16x8, w);
            if constexpr (VREG) vreg[s] = x;
            else vfrag[(wave * KS + s) * 64 + lane] = x;
        }
    }
    const uint16_t* qbase = (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh;
    const uint16_t* gbase = (const uint16_t*)p.dout + b * p.g_sb + h * p.g_sh;

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;

    // ---- steps: (entry e of the transposed row, 32-query sub-block sb) --------
    const int t0 = cload(p.p_row_ptr + kg), t1 = cload(p.p_row_ptr + kg + 1);
    struct Step {
        int e, sb, qt, mask0, mask1;
    };
    auto load_pair = [&](int e, Step& st) {
        const i32x4 v = cload((const i32x4*)(p.p_entries + e));
        st.qt = v[0];
        st.mask0 = v[1];
        st.mask1 = v[2];
    };
    auto first_step = [&]() {
        Step st{t0, 0, 0, -1, -1};
        if (t0 < t1) load_pair(t0, st);
        return st;
    };
    auto next_step = [&](Step st) {
        if (st.sb + 1 < nsub && st.qt * QBK + (st.sb + 1) * QS < N) {
            ++st.sb;
        } else {
            ++st.e;
            st.sb = 0;
            if (st.e < t1) load_pair(st.e, st);
        }
        return st;
    };

    // DMA rows of a step: slot = 64 * (wave + NW * i) + lane; slots [0, RSLOT)
    // are q rows, [RSLOT, 2 RSLOT) dout rows; (row, chunk) with CS chunks per
    // padded row, the pad chunk re-reading chunk 0.
    auto slot_rs = [&](int i) __attribute__((always_inline)) {
        const int slot = 64 * (wave + NW * i) + lane;
        return slot >= RSLOT ? slot - RSLOT : slot;
    };
    auto tokens = [&](Step st, int* tok) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int qp = min(st.qt * QBK + st.sb * QS + slot_rs(i) / CS, N - 1);
            tok[i] = p.perm ? gload(p.perm + qp) : qp;
        }
    };
    auto issue = [&](const int* tok, uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int blk = wave + NW * i;
            if (blk < NBLK) {
                const bool is_g = 64 * blk + lane >= RSLOT;
                const int ch = slot_rs(i) % CS;
                const uint32_t off = ch < CS - 1 ? 8 * ch : 0;
                const uint16_t* g = is_g ? gbase + ((uint32_t)tok[i] * (uint32_t)p.g_sn + off)
                                         : qbase + ((uint32_t)tok[i] * (uint32_t)p.q_sn + off);
                dma16(g, dst + blk * 512);
            }
        }
    };
    // lse / delta / mask words of a step, loaded into registers by wave 0 one
    // step ahead and written to LDS at the end of the previous step: lane t < 32
    // holds query t (stored at the accumulator position of query t), lane l
    // holds mask word (row l / 2, word l % 2) of each tile: all ones for a tile
    // without a mask, zero for a tile the query tile does not attend.  The
    // loads are unconditional from always-valid addresses (the query's token
    // clamped to the last one, fetched a step earlier still; the zero page for
    // tiles without a mask word) and every select waits for the store, after
    // the step's compute: a use right after a load would make wave 0 wait for
    // the rows just sent to LDS as well (the wait counter is in order).
    auto mask_src = [&](int mask, int sb) -> const uint32_t* {
        return mask >= 0 ? p.masks + ((int64_t)mask * QBK + sb * QS) * 2 : (const uint32_t*)p.zero;
    };
    auto part_src = [&](int mask, int sb) -> const uint32_t* {
        return mask >= 0 ? p.skip_masks + ((int64_t)mask * QBK + sb * QS) * 2 : (const uint32_t*)p.zero;
    };
    auto aux_valid = [&](Step st) { return st.qt * QBK + st.sb * QS + (lane & 31) < N; };
    auto aux_token = [&](Step st) -> int {
        const int qp = min(st.qt * QBK + st.sb * QS + (lane & 31), N - 1);
        return p.perm ? gload(p.perm + qp) : qp;
    };
    auto aux_fetch = [&](Step st, int tok, float* lr, float* dl, u32x4* mw) {
        *lr = gload(p.lse + (int64_t)bh * N + tok);
        *dl = gload(p.delta + (int64_t)bh * N + tok);
        (*mw)[0] = gload(mask_src(st.mask0, st.sb) + lane);
        (*mw)[1] = gload(mask_src(st.mask1, st.sb) + lane);
        if constexpr (BIAS) {
            (*mw)[2] = gload(part_src(st.mask0, st.sb) + lane);
            (*mw)[3] = gload(part_src(st.mask1, st.sb) + lane);
        }
    };
    auto aux_store = [&](Step st, float lr, float dl, u32x4 mw, float* aux) {
        // The lane index is passed through an empty asm statement so that the
        // compiler recomputes this step's LDS addresses (a few VALU
        // instructions) instead of keeping them across the walk: at 256
        // registers they would be spilled, and reloading a spill is a vector
        // memory access whose wait would also wait for the step's DMA.
        int lane_r = lane;
        asm volatile("" : "+v"(lane_r));
        const int t = lane_r & 31;
        const int a = t >> 4, rem = t & 15;
        const int pos = 16 * (rem & 1) + 8 * a + 4 * ((rem >> 1) & 1) + (rem >> 2);
        const bool valid = aux_valid(st);
        if (lane < 32) {
            aux[pos] = lse_log2(BIAS ? lr - p.lse_shift : lr, valid);
            aux[QS + pos] = valid ? dl : 0.f;
        }
        // a tile attended without a mask keeps every bit
        ((uint32_t*)aux)[2 * QS + lane_r] = st.mask0 == -1 ? ~0u : mw[0];
        ((uint32_t*)aux)[4 * QS + lane_r] = st.mask1 == -1 ? ~0u : mw[1];
        if constexpr (BIAS) {
            ((uint32_t*)aux)[6 * QS + lane_r] = mw[2];
            ((uint32_t*)aux)[8 * QS + lane_r] = mw[3];
        }
    };

    const int kappa = 16 * (l32 >> 4) + 2 * ((l32 >> 3) & 1) + ((l32 >> 2) & 1) + 4 * (l32 & 3);
    const int tr_base = (half + 4 * ((lane & 15) >> 2)) * ROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    auto compute = [&](Step st, const uint16_t* rl, const float* aux) {
        const int my_mask = wave >= 2 ? st.mask1 : st.mask0;   // wave-uniform
        if (my_mask == NA_MASK_NONE) return;   // this wave's tile is not attended by the step
        const uint16_t* ql = rl;
        const uint16_t* gl = rl + QS * ROW;
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
        {
            const uint16_t* qr = ql + kappa * ROW + 8 * half;
            const uint16_t* gr = gl + kappa * ROW + 8 * half;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qr + 16 * ks), kf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(gr + 16 * ks),
                                                             __builtin_bit_cast(bf16x8, VREG ? vreg[ks] : vfrag[(wave * KS + ks) * 64 + lane]), dp, 0,
                                                             0, 0);
            }
        }
        const uint32_t* mrows = (const uint32_t*)aux + 2 * QS + (wave >= 2 ? 2 * QS : 0);
        const uint32_t* prows = (const uint32_t*)aux + 6 * QS + (wave >= 2 ? 2 * QS : 0);
        const bool masked = my_mask >= 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 lv = *(const f32x4*)(aux + 16 * half + 4 * i);
            const f32x4 dl = *(const f32x4*)(aux + QS + 16 * half + 4 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * i + j;
                float sr = s[r];
                if constexpr (BIAS) {
                    if (masked) {  // partners outside the window carry the extra log-prior
                        const int q = 16 * (r / 8) + 2 * ((r / 4) % 2) + half + 4 * (r % 4);
                        sr += (prows[2 * q + (wave & 1)] >> l32) & 1u ? p.skip_bias : 0.f;
                    }
                }
                float pr = fast_exp2(__builtin_fmaf(sr, c, -lv[j]));
                if (masked) {
                    const int q = 16 * (r / 8) + 2 * ((r / 4) % 2) + half + 4 * (r % 4);
                    pr = (mrows[2 * q + (wave & 1)] >> l32) & 1u ? pr : 0.f;
                }
                s[r] = pr;
                dp[r] = pr * (dp[r] - dl[j]);
            }
        }
        // dv^T += dout^T P, dk^T += Q^T dS: 16 queries per step
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int r0 = 8 * ks;
            const bf16x8 bp = cvt8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4], s[r0 + 5], s[r0 + 6],
                                   s[r0 + 7]);
            const bf16x8 bd = cvt8(dp[r0], dp[r0 + 1], dp[r0 + 2], dp[r0 + 3], dp[r0 + 4], dp[r0 + 5],
                                   dp[r0 + 6], dp[r0 + 7]);
            const uint16_t* gr = gl + tr_base + 16 * ks * ROW;
            const uint16_t* qr = ql + tr_base + 16 * ks * ROW;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x4 glo = lds_read_tr(gr + 32 * db);
                const bf16x4 ghi = lds_read_tr(gr + 2 * ROW + 32 * db);
                dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7), bp, dv[db], 0, 0, 0);
                const bf16x4 qlo = lds_read_tr(qr + 32 * db);
                const bf16x4 qhi = lds_read_tr(qr + 2 * ROW + 32 * db);
                dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), bd, dk[db], 0, 0, 0);
            }
        }
    };

    // ---- pipelined walk: step t computes from buffer t % 2 while step t+1's
    // rows stream into the other; tokens are fetched two steps ahead -----------
    Step cur = first_step();
    if (cur.e < t1) {
        Step nx = next_step(cur);
        int tok[BPW];
        tokens(cur, tok);
        issue(tok, rows0);
        float lr, dl;
        u32x4 mw = {0u, 0u, 0u, 0u};
        int atok = 0;   // wave 0: the query token of step nx for lse / delta
        if (wave == 0) {
            aux_fetch(cur, aux_token(cur), &lr, &dl, &mw);
            aux_store(cur, lr, dl, mw, aux0);
        }
        int tok_n[BPW];
        if (nx.e < t1) {
            tokens(nx, tok_n);
            if (wave == 0) atok = aux_token(nx);
        }
        auto step = [&](const uint16_t* rl, const float* al, uint16_t* rn, float* an) {
            wait_vmem();
            __syncthreads();
            const Step nn = nx.e < t1 ? next_step(nx) : nx;
            if (nx.e < t1) {
                issue(tok_n, rn);
                if (wave == 0) aux_fetch(nx, atok, &lr, &dl, &mw);
                if (nn.e < t1) {
                    tokens(nn, tok_n);
                    if (wave == 0) atok = aux_token(nn);
                }
            }
            compute(cur, rl, al);
            if (nx.e < t1 && wave == 0) aux_store(nx, lr, dl, mw, an);
            cur = nx;
            nx = nn;
        };
        while (true) {
            step(rows0, aux0, rows1, aux1);
            if (cur.e >= t1) break;
            step(rows1, aux1, rows0, aux0);
            if (cur.e >= t1) break;
        }
    }
    wait_vmem();
    if (!kvalid) return;
    store_rows_t<DB>((uint16_t*)p.dk + b * p.dk_sb + h * p.dk_sh + (int64_t)ktok * p.dk_sn, dk, p.scale,
                     half);
    store_rows_t<DB>((uint16_t*)p.dv + b * p.dv_sb + h * p.dv_sh + (int64_t)ktok * p.dv_sn, dv, 1.f, half);
}

}  // namespace

bool na_bwd_supported(int dtype, int head_dim, int q_block, int kv_block) {
    return dtype == NA_BF16 && (head_dim == 64 || head_dim == 128) && kv_block == NA_KV_BLOCK_BF16 &&
           (q_block == 128 || q_block == 256);
}

namespace {

template <int D, bool BIAS>
int launch_bwd(const NaBwdParams& p, bool with_delta, hipStream_t st) {
    const int64_t rows = (int64_t)p.batch * p.heads * p.n_tokens;
    const dim3 gd((unsigned)((rows * (D / 8) + 255) / 256));
    const dim3 gq((unsigned)((int64_t)p.n_q_tiles * p.batch * p.heads));
    const dim3 gk((unsigned)((int64_t)((p.n_kv_tiles + 1) / 2) * p.batch * p.heads));
    if (with_delta) hipLaunchKernelGGL((bwd_delta<D>), gd, dim3(256), 0, st, p);
    if (p.q_block == 256)
        hipLaunchKernelGGL((attn_bwd_dq<D, 8, BIAS>), gq, dim3(512), 0, st, p);
    else
        hipLaunchKernelGGL((attn_bwd_dq<D, 4, BIAS>), gq, dim3(256), 0, st, p);
    hipLaunchKernelGGL((attn_bwd_dkdv<D, BIAS>), gk, dim3(256), 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace

int na_bwd_launch(const NaBwdParams& p, int head_dim, bool fusion, bool with_delta, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (head_dim == 128)
        return fusion ? launch_bwd<128, true>(p, with_delta, st) : launch_bwd<128, false>(p, with_delta, st);
    if (head_dim == 64)
        return fusion ? launch_bwd<64, true>(p, with_delta, st) : launch_bwd<64, false>(p, with_delta, st);
    return (int)hipErrorInvalidValue;
}

// ---- fixed device scratch of na_backward_noalloc ----------------------------
// The delta rows (fp32 [B][H][N]) of the no-allocation backward live in this
// array of the code object's static data: one copy per GPU, at its own address
// on each, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in): it takes the device
// address from hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) float scratch[NA_BACKWARD_NOALLOC_MAX_BYTES / sizeof(float)];

int na_bwd_scratch(void** ptr, size_t* bytes) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!addr) return (int)hipErrorInvalidSymbol;
        per_device[dev] = addr;
    }
    *ptr = per_device[dev];
    *bytes = sizeof(scratch);
    return 0;
}
