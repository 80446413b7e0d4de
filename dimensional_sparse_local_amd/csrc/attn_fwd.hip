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

#include "attn_common.h"

namespace {

// ---------------------------------------------------------------------------
// bf16: NW waves of 32 queries each (query tile 32*NW), key/value tile 64.
//
// Two waves share every SIMD (<= 256 registers each), so the MFMA phase of one
// overlaps the softmax phase of the other.  At D = 64 (128 registers) four
// waves share a SIMD, so up to four workgroups per CU keep K/V requests in
// flight for the short CSR rows of small windows.  K and V tiles (and the mask
// rows of a masked tile) travel from HBM/L2 straight into LDS (global_load_lds,
// 16 bytes per lane, no register staging) into two statically selected
// buffers: while tile e is computed from one buffer, tile e+1 streams into the
// other.  The gather addresses are prepared ahead: the CSR entry of tile e+3
// and the token indices of tile e+2 are fetched while tile e is computed, so
// no dependent load stalls a step.
//
// LDS rows of K and V are padded by one 16-byte chunk (row stride D + 8
// elements); the pad slot re-reads the row's first chunk, so one DMA block of
// 64 lanes covers 64 consecutive (row, chunk) slots and K and V share one slot
// -> row map.  Both operand reads are bank-conflict free at this stride: the K
// operand reads one chunk from each of 16 consecutive rows per 16-lane phase,
// and each V^T transpose read takes rows {0, 2, 8, 10} or {1, 3, 9, 11} (+4
// per half, +16 per step) of the tile, whose 32-byte segments fall on disjoint
// banks; the P^T operand slots follow the same row order.
//
// Online softmax in the log2 domain against a per-row reference maximum that
// moves only when it must (see kSumLog2).
// ---------------------------------------------------------------------------
template <int D, int NW, bool BIAS = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D == 64 && NW >= 4 && !BIAS ? 4 : 2,
                                   D == 64 && NW >= 4 && !BIAS ? 4 : 2)))
void attn_fwd_bf16(NaAttnParams p) {
    constexpr int KV = NA_KV_BLOCK_BF16;
    constexpr int QB = 32 * NW;
    constexpr int MP = BIAS ? 2 : 1;             // mask planes: keep (and fixed fusion's partners)
    constexpr int MB = (QB * 8 + 1023) / 1024;   // 1 KB DMA blocks per mask plane
    constexpr int ROW = D + 8;                   // padded LDS row (elements)
    constexpr int CS = D / 8 + 1;                // 16-byte slots per padded row
    constexpr int TILE = KV * ROW;               // LDS elements per tensor tile
    constexpr int NI = CS;                       // 1 KB DMA blocks per tensor tile (64*CS slots)
    constexpr int IPW = (NI + NW - 1) / NW;      // DMA blocks per wave (the last may be idle)
    constexpr int KS = D / 16;                   // QK reduction steps
    constexpr int DB = D / 32;                   // PV output blocks

    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
    // mask rows of the tile (two 32-key words per query row and plane), DMA'd
    // with K and V when the tile carries a mask
    __shared__ __attribute__((aligned(1024))) u32x2 m_lds0[MP][QB];
    __shared__ __attribute__((aligned(1024))) u32x2 m_lds1[MP][QB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
    const int half = lane >> 5, l32 = lane & 31;

    // whole tile, or one share of a tail tile's walk (split tail; never with
    // the fixed-fusion bias or the fused partner branch)
    const bool part_mode = (int)blockIdx.x >= p.n_main;
    const int part = (int)blockIdx.x - p.n_main;
    const int wg = part_mode ? p.n_main + part / p.n_split : xcd_remap(blockIdx.x, p.n_main);
    const int qt = tile_of(wg, p.n_q_tiles, p.q_desc);
    const int bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;
    const float c = p.scale_log2;

    // ---- this lane's query -------------------------------------------------
    const int qpos = qt * QB + wave * 32 + l32;
    const bool qvalid = qpos < N;
    const int qtok = qvalid ? (p.perm ? p.perm[qpos] : qpos) : 0;
    bf16x8 qf[KS];
    {
        const uint16_t* qrow =
            (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qtok * p.q_sn;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qvalid) w = *(const u32x4*)(qrow + 16 * s + 8 * half);
            qf[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const uint16_t* kbase = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh;
    const uint16_t* vbase = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh;
    // this lane's row of a tile mask (two 32-key words)
    const int mrow = wave * 32 + l32;

    // DMA block j = wave + NW*i moves slots 64*j .. 64*j+63 of a tile; lane t
    // moves slot 64*j + t = (row, chunk) with CS slots per row; chunk CS-1 is
    // the row's pad and re-reads chunk 0 (never read back), so every slot has a
    // real source.  Recomputed where used (CS is a compile-time constant).
    auto dma_row = [&](int i) { return (64 * (wave + NW * i) + lane) / CS; };
    auto dma_cb = [&](int i) {
        const uint32_t ch = (64 * (wave + NW * i) + lane) % CS;
        return ch < CS - 1 ? 16u * ch : 0u;
    };
    // Token of the row this lane moves in each of its DMA blocks, fetched one
    // step ahead.  Rows past the last token (the ragged last tile) are clamped
    // to the last token: the tile's mask excludes those keys, so their scores
    // are -inf and their probabilities exactly 0.  Its value is not used
    // before the DMA is issued, so fetching it never waits.
    auto tokens = [&](NaEntry entry, int* tok) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int kp = min(entry.kt * KV + dma_row(i), N - 1);
            tok[i] = p.perm ? gload(p.perm + kp) : kp;
        }
    };
    // Sources as a uniform base plus a 32-bit byte offset (a (batch, head)
    // slice spans fewer than 2^31 elements, checked on the host).
    const char* kb8 = (const char*)kbase;
    const char* vb8 = (const char*)vbase;
    const uint32_t k_rb = 2u * (uint32_t)p.k_sn, v_rb = 2u * (uint32_t)p.v_sn;
    auto issue = [&](NaEntry entry, const int* tok, uint16_t* kl, uint16_t* vl, u32x2 (*ml)[QB]) {
        if (entry.mask >= 0 && wave < MB * MP) {   // mask rows: 128 per block, two per lane
            const int plane = wave / MB, row = 128 * (wave % MB) + 2 * lane;
            const uint32_t* src = plane == 0 ? p.masks : p.skip_masks;
            if (row < QB) dma16(src + ((int64_t)entry.mask * QB + row) * 2, &ml[plane][row - 2 * lane]);
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int blk = wave + NW * i;
            if (blk < NI) {  // wave-uniform
                dma16(kb8 + ((uint32_t)tok[i] * k_rb + dma_cb(i)), kl + blk * 512);
                dma16(vb8 + ((uint32_t)tok[i] * v_rb + dma_cb(i)), vl + blk * 512);
            }
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_ref = kNegInf;   // reference maximum (log2 domain) of O and l
    float l_run = 0.f;

    // Key order inside a 32-key block.  MFMA row m of S^T = K Q^T is fed by
    // key kappa(m) = 16*(m/16) + 2*(m/8 % 2) + (m/4 % 2) + 4*(m % 4), so that
    // the accumulator elements r of half-wave h hold keys
    //     16*(r/8) + 2*(r/4 % 2) + h + 4*(r % 4)
    // and each group of 4 consecutive elements holds 4 keys spaced 4 apart:
    // rows whose 64-byte segments fall on disjoint LDS banks at the padded
    // stride, for both the K reads and the V^T transpose reads.
    const int kappa = 16 * (l32 >> 4) + 2 * ((l32 >> 3) & 1) + ((l32 >> 2) & 1) + 4 * (l32 & 3);
    // V^T transpose reads: in 16-lane group g = lane/16 the source lane
    // s = lane%16 supplies slot s/4: row 16*ks + half + 4*(s/4) (first read,
    // elements r0..r0+3) or + 2 (second read, r0+4..r0+7), element column
    // 32*db + 16*(g%2) + 4*(s%4).
    const int tr_base = (half + 4 * ((lane & 15) >> 2)) * ROW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // S^T = K Q^T for the two 32-key halves of the tile, masked where the tile
    // is partial (or runs past the last key).
    auto scores = [&](NaEntry entry, const u32x2 (*ml)[QB], const uint16_t* kl, f32x16* s) {
        // All KS fragments of the first half are requested up front; each MFMA
        // of the first half is then followed by the request for the matching
        // fragment of the second half, so LDS latency hides behind MFMA work.
#pragma unroll
        for (int r = 0; r < 16; ++r) s[0][r] = s[1][r] = 0.f;
        {
            const uint16_t* kr0 = kl + kappa * ROW + 8 * half;
            const uint16_t* kr1 = kr0 + 32 * ROW;
            bf16x8 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const bf16x8*)(kr0 + 16 * ks);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s[0], 0, 0, 0);
                kf[ks] = *(const bf16x8*)(kr1 + 16 * ks);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s[1], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);   // KS LDS reads
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);   // KS MFMAs
        }
        // element mask (partial tiles and tiles past the last key only): score
        // (kb, r) is key 32*kb + 16*(r/8) + 2*(r/4 % 2) + half + 4*(r % 4)
        if (entry.mask >= 0) {
            const u32x2 mk = ml[0][mrow];
            const uint32_t w0 = mk[0] >> half, w1 = mk[1] >> half;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int bit = 16 * (r / 8) + 2 * ((r / 4) % 2) + 4 * (r % 4);
                s[0][r] = keep_if(w0, bit, s[0][r]);
                s[1][r] = keep_if(w1, bit, s[1][r]);
            }
            if constexpr (BIAS) {
                // fixed fusion: partners outside the window carry the extra
                // log-prior, as an offset of the raw dot product
                const u32x2 bk = ml[1][mrow];
                const uint32_t b0 = bk[0] >> half, b1 = bk[1] >> half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int bit = 16 * (r / 8) + 2 * ((r / 4) % 2) + 4 * (r % 4);
                    s[0][r] += ((b0 >> bit) & 1u) ? p.skip_bias : 0.f;
                    s[1][r] += ((b1 >> bit) & 1u) ? p.skip_bias : 0.f;
                }
            }
        }
    };
    // s <- 2^(c s - m_ref), fp32; returns this lane's sum of them.  A row with
    // no reference yet (m_ref = -inf) takes 0 here and is redone below.
    auto probs = [&](f32x16* s, uint32_t live) {
        const float neg_m = m_ref == kNegInf ? 0.f : -m_ref;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if ((live >> kb) & 1u) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, neg_m));
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
            }
        }
        return tile_sum32(s[0], s[1]);
    };
    // On a partial tile a 32-key block that no query of this wave attends
    // skips its exponentials and P.V products, and the wave skips the whole
    // tile when both are.
    auto compute = [&](NaEntry entry, const u32x2 (*ml)[QB], const uint16_t* kl, const uint16_t* vl) {
        uint32_t live = 3u;
        if (entry.mask >= 0) {
            const u32x2 any = ml[0][mrow];   // the keep plane holds every attended key
            live = (__builtin_amdgcn_ballot_w64(any[0] != 0u) ? 1u : 0u) |
                   (__builtin_amdgcn_ballot_w64(any[1] != 0u) ? 2u : 0u);
            if (live == 0u) return;
        }
        f32x16 s[2];
        scores(entry, ml, kl, s);
        // Online softmax against a reference maximum that moves only when it
        // must: the probabilities are taken against the row's current
        // reference, and the exact tile maximum is formed only if a row has no
        // reference yet (taken from these scores) or a lane's sum of this
        // tile's probabilities (which bounds each of them) passes 2^kSumLog2
        // (the wave then recomputes the scores the exponentials overwrote).
        // The wave moves every row's reference to max(reference, tile
        // maximum), rescaling O and l; the result is exact after the final
        // division by l either way.
        float ts = 0.f;
        bool need_max = __builtin_amdgcn_ballot_w64(m_ref == kNegInf) != 0;
        if (!need_max) {
            ts = probs(s, live);
            if (__builtin_amdgcn_ballot_w64(!(ts <= kSumMax))) {
                need_max = true;
                scores(entry, ml, kl, s);
            }
        }
        if (need_max) {
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
            const float m_new = fmaxf(m_ref, halves_max(mx) * c);   // both halves of a row agree
            if (m_new > m_ref) {
                const float alpha = fast_exp2(m_ref - m_new);   // 0 when m_ref = -inf
                m_ref = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            }
            ts = probs(s, live);
        }
        // the row sum takes the fp32 probabilities, before their rounding to
        // bf16 for P V, so lse carries fp32 rounding only
        l_run += ts;
        // O^T += V^T P^T, 16 keys per step.  Step ks covers accumulator
        // elements r0 = 8*(ks%2) .. r0+7 of score block ks/2: slot e of half h
        // is key 16*ks + 2*(e/4) + h + 4*(e%4), the row the transpose reads
        // deliver for that slot.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (!((live >> (ks / 2)) & 1u)) continue;
            const f32x16& sv = s[ks / 2];
            const int r0 = 8 * (ks % 2);
            const bf16x8 bp = cvt8(sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3], sv[r0 + 4],
                                   sv[r0 + 5], sv[r0 + 6], sv[r0 + 7]);
            const uint16_t* vr = vl + tr_base + 16 * ks * ROW;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x4 lo = lds_read_tr(vr + 32 * db);
                const bf16x4 hi = lds_read_tr(vr + 2 * ROW + 32 * db);
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[db], 0, 0, 0);
            }
        }
    };

    // ---- pipelined walk over the CSR row ------------------------------------
    // Entering step e: tile e (K, V and its mask rows) is in flight to (or in)
    // its LDS buffers, ent_a..c are the entries of tiles e..e+2 and tok_n the
    // tokens of tile e+1.
    int e0 = cload(p.row_ptr + qt), e1 = cload(p.row_ptr + qt + 1);
    if (part_mode) {
        const int len = e1 - e0, j = part % p.n_split;
        e1 = e0 + (len * (j + 1)) / p.n_split;
        e0 = e0 + (len * j) / p.n_split;
    }
    const NaEntry none = {0, -1};
    NaEntry ent_a = none, ent_b = none, ent_c = none;
    int tok_n[IPW];
    if (e0 < e1) {
        ent_a = load_entry(p.entries + e0);
        if (e0 + 1 < e1) ent_b = load_entry(p.entries + e0 + 1);
        if (e0 + 2 < e1) ent_c = load_entry(p.entries + e0 + 2);
        int tok0[IPW];
        tokens(ent_a, tok0);
        issue(ent_a, tok0, k_lds0, v_lds0, m_lds0);
        if (e0 + 1 < e1) tokens(ent_b, tok_n);
    }
    auto step = [&](int e, const uint16_t* kl, const uint16_t* vl, const u32x2 (*ml)[QB], uint16_t* kn,
                    uint16_t* vn, u32x2 (*mn)[QB]) {
        wait_vmem();
        __syncthreads();
        if (e + 1 < e1) issue(ent_b, tok_n, kn, vn, mn);
        if (e + 2 < e1) tokens(ent_c, tok_n);
        const NaEntry ent_d = e + 3 < e1 ? load_entry(p.entries + e + 3) : none;
        compute(ent_a, ml, kl, vl);
        ent_a = ent_b;
        ent_b = ent_c;
        ent_c = ent_d;
    };
    for (int e = e0; e < e1; e += 2) {
        step(e, k_lds0, v_lds0, m_lds0, k_lds1, v_lds1, m_lds1);
        if (e + 1 < e1) step(e + 1, k_lds1, v_lds1, m_lds1, k_lds0, v_lds0, m_lds0);
    }

    // ---- epilogue -----------------------------------------------------------
    // A share of a split tile stores its unnormalised O (fp32), reference
    // maximum and row sum for the merge; a whole tile stores O / l and lse.
    const float l_tot = halves_sum(l_run);
    const bool share = !BIAS && part_mode;
    if (!share && !qvalid) return;
    const float inv = share ? 1.f : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    uint16_t* orow = (uint16_t*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)qtok * p.o_sn;
    const int64_t srow = (int64_t)part * QB + wave * 32 + l32;   // share mode: row of part_o
    // pi-Attention's separate softmax ("pi-Attention", Section 3.5, Eq. 15):
    // the softmax over this query's online partners x - pi (and x + pi; Eq. 9),
    // a separate distribution whose weighted value average is added to the
    // window's.  Each half-wave holds half of q (elements 16 s + 8 half ..
    // +7), so the partial dot products of the two halves are summed across
    // lanes l and l ^ 32; an absent partner reads a clamped row and gets
    // weight 0, so both halves always take part.
    // At D = 64 every load (key and value rows of both partners) is issued
    // first, so the tail pays one memory round trip; at D = 128 that many
    // registers would spill, and the value rows are read at the store.
    constexpr bool PRELOAD = D == 64;
    float pw[2] = {0.f, 0.f};
    const uint16_t* prow[2] = {vbase, vbase};
    uint2 pv[2][DB][4];   // PRELOAD: this lane's 4-element groups of the partners' value rows
    if constexpr (!BIAS) {
        if (p.sep_skip > 0) {   // uniform
            bool has[2];
            float z[2];
            // q . k over this lane's half of the head dimension (the explicit
            // (uint32_t) matters: hipcc miscompiles a bit_cast of a bare
            // vector element, giving every j word 0)
            auto half_dot = [&](const u32x4* kw) {
                float dot = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) {
                    const u32x4 qw = __builtin_bit_cast(u32x4, qf[s2]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)qw[j]),
                                                              __builtin_bit_cast(bf16x2, (uint32_t)kw[s2][j]),
                                                              dot, false);
                }
                return dot;
            };
            // partner t's row (sequence position x -/+ pi, clamped) and whether it exists
            auto partner = [&](int t, const uint16_t** krow) {
                const int x = t == 0 ? qpos - p.sep_skip : qpos + p.sep_skip;
                has[t] = t == 0 ? x >= 0 : (p.sep_both != 0 && x < N);
                const int xc = min(max(x, 0), N - 1);
                const int tok = p.perm ? p.perm[xc] : xc;
                *krow = kbase + (int64_t)tok * p.k_sn + 8 * half;
                prow[t] = vbase + (int64_t)tok * p.v_sn;
            };
            if constexpr (PRELOAD) {
                u32x4 kw[2][KS];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint16_t* krow;
                    partner(t, &krow);
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) kw[t][s2] = *(const u32x4*)(krow + 16 * s2);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            pv[t][db][g] = *(const uint2*)(prow[t] + 32 * db + 8 * g + 4 * half);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) z[t] = has[t] ? halves_sum(half_dot(kw[t])) * c : kNegInf;
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint16_t* krow;
                    partner(t, &krow);
                    u32x4 kw[KS];
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) kw[s2] = *(const u32x4*)(krow + 16 * s2);
                    z[t] = has[t] ? halves_sum(half_dot(kw)) * c : kNegInf;   // log2 domain
                }
            }
            const float m = fmaxf(z[0], z[1]);
            if (m > kNegInf) {
                const float e0 = has[0] ? fast_exp2(z[0] - m) : 0.f;
                const float e1 = has[1] ? fast_exp2(z[1] - m) : 0.f;
                const float il = 1.f / (e0 + e1);
                pw[0] = e0 * il;
                pw[1] = e1 * il;
            }
        }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * half;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = o[db][4 * g + i] * inv;
            if constexpr (!BIAS) {
                if (p.sep_skip > 0) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const uint2 vw = PRELOAD ? pv[t][db][g] : *(const uint2*)(prow[t] + d);
                        y[0] = __builtin_fmaf(pw[t], __builtin_bit_cast(float, vw.x << 16), y[0]);
                        y[1] = __builtin_fmaf(pw[t], __builtin_bit_cast(float, vw.x & 0xffff0000u), y[1]);
                        y[2] = __builtin_fmaf(pw[t], __builtin_bit_cast(float, vw.y << 16), y[2]);
                        y[3] = __builtin_fmaf(pw[t], __builtin_bit_cast(float, vw.y & 0xffff0000u), y[3]);
                    }
                }
            }
            if (share) {
                *(f32x4*)(p.part_o + srow * D + d) = f32x4{y[0], y[1], y[2], y[3]};
                continue;
            }
            const f32x2 x0 = {y[0], y[1]};
            const f32x2 x1 = {y[2], y[3]};
            const uint2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(x0, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(x1, bf16x2))};
            *(uint2*)(orow + d) = w;
        }
    if (share) {
        if (half == 0) *(f32x2*)(p.part_ml + 2 * srow) = f32x2{m_ref, l_tot};
        return;
    }
    if (p.lse && half == 0) {
        float lse = l_tot > 0.f ? (m_ref + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
        if constexpr (BIAS) lse += p.lse_shift;  // the log(alpha) common to every logit
        p.lse[(int64_t)bh * N + qtok] = lse;
    }
}

// ---------------------------------------------------------------------------
// bf16, 4 waves of 48 queries each (query tile 192), key/value tile 64, built
// on 16x16x32 MFMAs.  Each wave holds three 16-query blocks, so every K and V
// fragment read from LDS feeds three MFMAs: a third less LDS traffic per flop
// than 32 queries per wave, at the same two waves per SIMD.
//
// 16x16x32 layouts: A operand lane l holds row l%16 and reduction slots
// 8*(l/16) .. +7; B likewise for column l%16; the accumulator lane l holds
// column l%16 and rows 4*(l/16) .. +3.  Within a 16-key block, MFMA row m is
// fed by key pi(m) = 4*(m%4) + 2*(m/4 % 2) + m/8, so lane-group g holds keys
// 4*i + cg with cg = 2*(g%2) + g/2: the rows of each V^T transpose read are
// spaced two apart and the K reads of a 16-lane phase cover 16 distinct rows,
// which keeps both on distinct banks, at the padded stride (D = 64) and with
// the chunk permutation of the unpadded rows (D = 128).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const float y = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    return halves_max(y);
}
__device__ __forceinline__ float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return halves_sum(__builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]));
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_m16(NaAttnParams p) {
    constexpr int QBN = 3;                       // 16-query blocks per wave
    constexpr int QB = 16 * QBN * NW;            // 192 or 384
    constexpr int KV = NA_KV_BLOCK_BF16;
    // K and V tiles in LDS.  At D = 128 a row is 16 chunks of 16 bytes stored
    // unpadded, chunk j of row r at position j ^ (r % 16) of the row: the K
    // reads of a 16-lane phase (16 rows, one chunk each) and the transpose
    // reads of V (8 rows, 32 bytes each) then fall on distinct banks, and a
    // tile is 16 DMA blocks, two or four per wave.  Otherwise (D = 64) rows
    // are padded by one chunk (the pad slot re-reads chunk 0 and is never
    // read back).
    constexpr bool SWZ = D == 128;
    constexpr int ROW = SWZ ? D : D + 8;
    constexpr int CS = SWZ ? D / 8 : D / 8 + 1;   // 16-byte slots per row
    constexpr int TILE = KV * ROW;
    constexpr int NI = KV * CS / 64;              // 1 KB DMA blocks per tile
    constexpr int IPW = (NI + NW - 1) / NW;
    constexpr int KS = D / 32;                   // QK reduction steps
    constexpr int DB = D / 16;                   // PV output blocks

    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[TILE];
    // mask rows of the tile (two 32-key words per query row), DMA'd with K and V
    __shared__ __attribute__((aligned(1024))) u32x2 m_lds0[QB];
    __shared__ __attribute__((aligned(1024))) u32x2 m_lds1[QB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q16 = lane & 15, g = lane >> 4;
    const int cg = 2 * (g & 1) + (g >> 1);

    // whole tile, or one share of a tail tile's walk (split tail)
    const bool part_mode = (int)blockIdx.x >= p.n_main;
    const int part = (int)blockIdx.x - p.n_main;
    const int wg = part_mode ? p.n_main + part / p.n_split : xcd_remap(blockIdx.x, p.n_main);
    const int qt = tile_of(wg, p.n_q_tiles, p.q_desc);
    const int bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int N = p.n_tokens;
    const float c = p.scale_log2;

    // ---- this lane's three queries --------------------------------------------
    bf16x8 qf[QBN][KS];
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        const int qpos = qt * QB + wave * (16 * QBN) + 16 * qb + q16;
        const bool qvalid = qpos < N;
        const int qtok = qvalid ? (p.perm ? p.perm[qpos] : qpos) : 0;
        const uint16_t* qrow =
            (const uint16_t*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qtok * p.q_sn;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (qvalid) w = *(const u32x4*)(qrow + 32 * ks + 8 * g);
            qf[qb][ks] = __builtin_bit_cast(bf16x8, w);
        }
    }
    const uint16_t* kbase = (const uint16_t*)p.k + b * p.k_sb + h * p.k_sh;
    const uint16_t* vbase = (const uint16_t*)p.v + b * p.v_sb + h * p.v_sh;

    // ---- DMA of one key/value tile (as in the 32-query kernel) -----------------
    // slot -> (row, byte offset of the chunk); recomputed where used to save
    // registers (CS is a compile-time constant).  Rows past the last token are
    // clamped to it (masked keys, probability exactly 0).
    auto dma_row = [&](int i) { return (64 * (wave + NW * i) + lane) / CS; };
    auto dma_cb = [&](int i) {
        const int slot = 64 * (wave + NW * i) + lane;
        const uint32_t ch = (uint32_t)(slot % CS);
        if constexpr (SWZ) return 16u * (ch ^ ((uint32_t)(slot / CS) & 15u));
        else return ch < CS - 1 ? 16u * ch : 0u;
    };
    auto tokens = [&](NaEntry entry, int* tok) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int kp = min(entry.kt * KV + dma_row(i), N - 1);
            tok[i] = p.perm ? gload(p.perm + kp) : kp;
        }
    };
    const char* kb8 = (const char*)kbase;
    const char* vb8 = (const char*)vbase;
    const uint32_t k_rb = 2u * (uint32_t)p.k_sn, v_rb = 2u * (uint32_t)p.v_sn;
    auto issue = [&](NaEntry entry, const int* tok, uint16_t* kl, uint16_t* vl, u32x2* ml) {
        // the tile's mask rows: QB rows of 8 bytes, 1 KB (128 rows) per wave
        if (entry.mask >= 0 && wave < (QB * 8) / 1024 + 1) {
            const int row = 128 * wave + lane * 2;   // two 8-byte rows per lane
            if (row < QB)
                dma16(p.masks + ((int64_t)entry.mask * QB + row) * 2, ml + 128 * wave);
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int blk = wave + NW * i;
            if (blk < NI) {
                dma16(kb8 + ((uint32_t)tok[i] * k_rb + dma_cb(i)), kl + blk * 512);
                dma16(vb8 + ((uint32_t)tok[i] * v_rb + dma_cb(i)), vl + blk * 512);
            }
        }
    };
    f32x4 o[DB][QBN];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref[QBN], l_run[QBN];
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        m_ref[qb] = kNegInf;
        l_run[qb] = 0.f;
    }

    const int pim = q16;   // A-operand row of this lane inside a 16-key block
    const int pi = 4 * (pim & 3) + 2 * ((pim >> 2) & 1) + (pim >> 3);
    // element offsets inside a row: of this lane's K fragment for step ks (row
    // 32*hs + 16*kb + pi), and of its V^T transpose read for output block db
    // (row 32*hs + 16*j + vrow)
    auto kcol = [&](int ks) { return SWZ ? 8 * ((4 * ks + g) ^ pi) : 32 * ks + 8 * g; };
    const int vrow = 4 * (q16 >> 2) + cg;
    auto vcol = [&](int db) {
        return SWZ ? 8 * ((2 * db + ((q16 & 3) >> 1)) ^ vrow) + 4 * (q16 & 1) : 16 * db + 4 * (q16 & 3);
    };

    // S^T blocks of one 32-key half: keys 32*hs + 16*kb .. +15, queries of
    // block qb; masked where the tile is partial (or runs past the last key).
    auto scores = [&](int hs, NaEntry entry, const u32x2* ml, const uint16_t* kl, f32x4 (*s)[QBN]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            // k-step outer, one step of lookahead: fragments of both 16-key
            // blocks for step ks+1 load while the 6 MFMAs of step ks run
            const uint16_t* kr = kl + (32 * hs + pi) * ROW;
            bf16x8 a0 = *(const bf16x8*)(kr + kcol(0));
            bf16x8 a1 = *(const bf16x8*)(kr + 16 * ROW + kcol(0));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 n0 = a0, n1 = a1;
                if (ks + 1 < KS) {
                    n0 = *(const bf16x8*)(kr + kcol(ks + 1));
                    n1 = *(const bf16x8*)(kr + 16 * ROW + kcol(ks + 1));
                }
#pragma unroll
                for (int qb = 0; qb < QBN; ++qb) {
                    s[0][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[qb][ks], s[0][qb], 0, 0, 0);
                    s[1][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[qb][ks], s[1][qb], 0, 0, 0);
                }
                a0 = n0;
                a1 = n1;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // element mask: element i of block kb is key 32*hs + 16*kb + 4*i + cg
        if (entry.mask >= 0) {
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) {
                const uint32_t w = ml[wave * (16 * QBN) + 16 * qb + q16][hs] >> cg;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[kb][qb][i] = keep_if(w, 16 * kb + 4 * i, s[kb][qb][i]);
            }
        }
    };
    // s <- 2^(c s - m_ref) per query block, fp32; ts[qb] = this lane's sums.
    auto probs = [&](f32x4 (*s)[QBN], float* ts) {
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
            const float neg_m = m_ref[qb] == kNegInf ? 0.f : -m_ref[qb];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[kb][qb][i] = fast_exp2(__builtin_fmaf(s[kb][qb][i], c, neg_m));
            ts[qb] = ((s[0][qb][0] + s[0][qb][1]) + (s[0][qb][2] + s[0][qb][3])) +
                     ((s[1][qb][0] + s[1][qb][1]) + (s[1][qb][2] + s[1][qb][3]));
        }
    };

    // One K/V tile; mid() runs once the first half's scores are in registers
    // (the walk issues the next tile's DMA there, so its LDS writes overlap
    // the softmax and P.V products rather than this tile's K reads).
    //
    // With four waves (192-query tiles), a wave skips a half of a partial tile
    // whose 32 keys none of its queries attends (bit hs of `live`); at eight
    // waves the same test measured slower on full-tile maps and is compiled
    // out.
    auto compute = [&](NaEntry entry, const u32x2* ml, const uint16_t* kl, const uint16_t* vl,
                       auto mid) {
        uint32_t live = 3u;
        if (NW == 4 && entry.mask >= 0) {
            u32x2 any = ml[wave * (16 * QBN) + q16];
#pragma unroll
            for (int qb = 1; qb < QBN; ++qb) any |= ml[wave * (16 * QBN) + 16 * qb + q16];
            live = (__builtin_amdgcn_ballot_w64(any[0] != 0u) ? 1u : 0u) |
                   (__builtin_amdgcn_ballot_w64(any[1] != 0u) ? 2u : 0u);
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {   // two 32-key halves of the tile
            const bool run = (live >> hs) & 1u;
            f32x4 s[2][QBN];
            if (run) scores(hs, entry, ml, kl, s);
            if (hs == 0) mid();
            if (!run) continue;

            // online softmax against each row's reference maximum, which moves
            // only for a row with none yet or a lane sum past 2^kSumLog2 (the
            // wave then recomputes the half's scores and takes exact maxima)
            float ts[QBN];
            probs(s, ts);
            bool redo = false;
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) redo = redo || m_ref[qb] == kNegInf || !(ts[qb] <= kSumMax);
            if (__builtin_amdgcn_ballot_w64(redo)) {
                scores(hs, entry, ml, kl, s);
#pragma unroll
                for (int qb = 0; qb < QBN; ++qb) {
                    float mx = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), fmaxf(s[0][qb][2], s[0][qb][3]));
                    mx = fmaxf(mx, fmaxf(fmaxf(s[1][qb][0], s[1][qb][1]), fmaxf(s[1][qb][2], s[1][qb][3])));
                    const float m_new = fmaxf(m_ref[qb], quad_max(mx) * c);   // the row's four lanes agree
                    if (m_new > m_ref[qb]) {
                        const float alpha = fast_exp2(m_ref[qb] - m_new);   // 0 when m_ref = -inf
                        m_ref[qb] = m_new;
                        l_run[qb] *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[db][qb][i] *= alpha;
                    }
                }
                probs(s, ts);
            }
            // fp32 row sums of the probabilities before their bf16 rounding
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) l_run[qb] += ts[qb];
            // P^T operands: slot j = 4*kb + i of lane-group g is key 32*hs + 16*kb + 4*i + cg
            bf16x8 bp[QBN];
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) {
                bp[qb] = cvt8(s[0][qb][0], s[0][qb][1], s[0][qb][2], s[0][qb][3], s[1][qb][0],
                              s[1][qb][1], s[1][qb][2], s[1][qb][3]);
            }
            // O^T += V^T P^T: the transpose reads give slot j' of group g the
            // row 32*hs + 4*j' + cg (first read) or + 16 (second read)
            const uint16_t* vr = vl + (32 * hs + vrow) * ROW;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x4 lo = lds_read_tr(vr + vcol(db));
                const bf16x4 hi = lds_read_tr(vr + 16 * ROW + vcol(db));
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < QBN; ++qb)
                    o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[qb], o[db][qb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- pipelined walk over the CSR row (as in the 32-query kernel) -----------
    int e0 = cload(p.row_ptr + qt), e1 = cload(p.row_ptr + qt + 1);
    if (part_mode) {
        const int len = e1 - e0, j = part % p.n_split;
        e1 = e0 + (len * (j + 1)) / p.n_split;
        e0 = e0 + (len * j) / p.n_split;
    }
    const NaEntry none = {0, -1};
    NaEntry ent_a = none, ent_b = none, ent_c = none;
    int tok_n[IPW];
    if (e0 < e1) {
        ent_a = load_entry(p.entries + e0);
        if (e0 + 1 < e1) ent_b = load_entry(p.entries + e0 + 1);
        if (e0 + 2 < e1) ent_c = load_entry(p.entries + e0 + 2);
        int tok0[IPW];
        tokens(ent_a, tok0);
        issue(ent_a, tok0, k_lds0, v_lds0, m_lds0);
        if (e0 + 1 < e1) tokens(ent_b, tok_n);
    }
    auto step = [&](int e, const uint16_t* kl, const uint16_t* vl, const u32x2* ml, uint16_t* kn,
                    uint16_t* vn, u32x2* mn) {
        wait_vmem();
        __syncthreads();
        const NaEntry ent_d = e + 3 < e1 ? load_entry(p.entries + e + 3) : none;
        compute(ent_a, ml, kl, vl, [&]() {
            if (e + 1 < e1) issue(ent_b, tok_n, kn, vn, mn);
            if (e + 2 < e1) tokens(ent_c, tok_n);
        });
        ent_a = ent_b;
        ent_b = ent_c;
        ent_c = ent_d;
    };
    for (int e = e0; e < e1; e += 2) {
        step(e, k_lds0, v_lds0, m_lds0, k_lds1, v_lds1, m_lds1);
        if (e + 1 < e1) step(e + 1, k_lds1, v_lds1, m_lds1, k_lds0, v_lds0, m_lds0);
    }

    // ---- epilogue -----------------------------------------------------------------
    if (part_mode) {   // unnormalised share: O, reference maximum, row sum
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
            const float l_tot = quad_sum(l_run[qb]);
            const int row = wave * (16 * QBN) + 16 * qb + q16;
            float* po = p.part_o + ((int64_t)part * QB + row) * D + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db) *(f32x4*)(po + 16 * db) = o[db][qb];
            if (g == 0)
                *(f32x2*)(p.part_ml + 2 * ((int64_t)part * QB + row)) = f32x2{m_ref[qb], l_tot};
        }
        return;
    }
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        const float l_tot = quad_sum(l_run[qb]);
        const int qpos = qt * QB + wave * (16 * QBN) + 16 * qb + q16;
        if (qpos >= N) continue;
        const int qtok = p.perm ? p.perm[qpos] : qpos;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = (uint16_t*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)qtok * p.o_sn;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f32x2 x0 = {o[db][qb][0] * inv, o[db][qb][1] * inv};
            const f32x2 x1 = {o[db][qb][2] * inv, o[db][qb][3] * inv};
            const uint2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(x0, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(x1, bf16x2))};
            *(uint2*)(orow + 16 * db + 4 * g) = w;
        }
        if (p.lse && g == 0) {
            const float lse = l_tot > 0.f ? (m_ref[qb] + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(int64_t)bh * N + qtok] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// Split tail: merge the n_split shares of each tail tile's walk.  Share j of
// row i holds O_j = sum 2^(c s - m_j) v and l_j = sum 2^(c s - m_j) over its
// keys; with M = max m_j over shares that saw a key,
//     out_i = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j,
//     lse_i = (M + log2 sum_j 2^(m_j - M) l_j) ln 2,
// the same result as one walk over all the keys.  Four columns per thread.
// ---------------------------------------------------------------------------
template <int D, int QB>
__global__ __launch_bounds__(256) void attn_fwd_combine(NaAttnParams p) {
    constexpr int TPR = D / 4;         // threads per row
    constexpr int RPB = 256 / TPR;     // rows per block
    const int gr = blockIdx.x * RPB + (int)threadIdx.x / TPR;
    const int c4 = (int)threadIdx.x % TPR;
    if (gr >= (p.n_wg - p.n_main) * QB) return;
    const int tt = gr / QB, row = gr % QB;
    const int wg = p.n_main + tt;
    const int qt = tile_of(wg, p.n_q_tiles, p.q_desc), bh = wg / p.n_q_tiles;
    const int b = bh / p.heads, h = bh % p.heads;
    const int qpos = qt * QB + row;
    if (qpos >= p.n_tokens) return;
    const int64_t first = (int64_t)tt * p.n_split * QB + row;   // share 0 of this row
    float M = kNegInf;
    for (int j = 0; j < p.n_split; ++j) {
        const f32x2 ml = *(const f32x2*)(p.part_ml + 2 * (first + (int64_t)j * QB));
        if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.n_split; ++j) {
        const int64_t r = first + (int64_t)j * QB;
        const f32x2 ml = *(const f32x2*)(p.part_ml + 2 * r);
        if (!(ml[1] > 0.f)) continue;
        const float w = fast_exp2(ml[0] - M);
        L += w * ml[1];
        const f32x4 oj = *(const f32x4*)(p.part_o + r * D + 4 * c4);
        acc += w * oj;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int qtok = p.perm ? p.perm[qpos] : qpos;
    uint16_t* orow = (uint16_t*)p.out + b * p.o_sb + h * p.o_sh + (int64_t)qtok * p.o_sn;
    const f32x2 x0 = {acc[0] * inv, acc[1] * inv};
    const f32x2 x1 = {acc[2] * inv, acc[3] * inv};
    const uint2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(x0, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(x1, bf16x2))};
    *(uint2*)(orow + 4 * c4) = w;
    if (p.lse && c4 == 0)
        p.lse[(int64_t)bh * p.n_tokens + qtok] =
            L > 0.f ? (M + __builtin_log2f(L)) * kLn2 : kNegInf;
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
        const NaEntry entry = p.entries[e];
        const int kt = entry.kt;
        // stage the tile: lane handles key rows lane%32, half of the columns each
        for (int row = 0; row < KV; ++row) {
            const int kp = kt * KV + row;
            const int tok = kp < N ? (p.perm ? p.perm[kp] : kp) : -1;
            for (int c = lane; c < D; c += 64) {
                k_lds[row * ROW + c] = tok >= 0 ? kbase[(int64_t)tok * p.k_sn + c] : 0.f;
                v_lds[row * ROW + c] = tok >= 0 ? vbase[(int64_t)tok * p.v_sn + c] : 0.f;
            }
        }
        // this lane's mask row (bit k = key k of the tile attended)
        const uint32_t mk = entry.mask >= 0 ? p.masks[(int64_t)entry.mask * 32 + l32] >> (4 * half)
                                            : 0u;
        __syncthreads();

        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(k_lds[l32 * ROW + 2 * ks + half], qf[ks], s, 0,
                                                     0, 0);
        float mt = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = s[r] * p.scale_log2;
            if (entry.mask >= 0) x = keep_if(mk, 8 * (r / 4) + (r % 4), x);
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

bool na_attn_supported(int dtype, int head_dim, int q_block, int kv_block, bool fusion) {
    if (fusion)  // the logit bias exists in the 32-query-per-wave bf16 kernels
        return dtype == NA_BF16 && (head_dim == 64 || head_dim == 128) &&
               kv_block == NA_KV_BLOCK_BF16 &&
               (q_block == 128 || q_block == 256 || (q_block == 64 && head_dim == 64));
    if (dtype == NA_BF16)
        return (head_dim == 64 || head_dim == 128) && kv_block == NA_KV_BLOCK_BF16 &&
               (q_block == 128 || q_block == 192 || q_block == 256 ||
                (q_block == 64 && head_dim == 64) || (q_block == 384 && head_dim == 128));
    if (dtype == NA_F32)
        return (head_dim == 32 || head_dim == 64) && kv_block == NA_KV_BLOCK_F32 &&
               q_block == NA_Q_BLOCK_F32;
    return false;
}

namespace {

// The kernel (and its block size) of a launch that has the split-walk mode,
// or false.
bool split_kernel(int dtype, int head_dim, int q_block, bool fusion, const void** fn, int* threads) {
    if (dtype != NA_BF16 || fusion) return false;
    if (head_dim == 64 && q_block == 64)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16<64, 2>), *threads = 128;
    else if (head_dim == 64 && q_block == 128)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16<64, 4>), *threads = 256;
    else if (head_dim == 64 && q_block == 256)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16<64, 8>), *threads = 512;
    else if (head_dim == 128 && q_block == 128)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16<128, 4>), *threads = 256;
    else if (head_dim == 128 && q_block == 256)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16<128, 8>), *threads = 512;
    else if (head_dim == 128 && q_block == 384)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16_m16<128, 8>), *threads = 512;
    else if (head_dim == 128 && q_block == 192)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16_m16<128, 4>), *threads = 256;
    else if (head_dim == 64 && q_block == 192)
        *fn = reinterpret_cast<const void*>(&attn_fwd_bf16_m16<64, 4>), *threads = 256;
    else
        return false;
    return true;
}

}  // namespace

int na_attn_split_capacity(int dtype, int head_dim, int q_block, bool fusion) {
    const void* fn = nullptr;
    int threads = 0;
    if (!split_kernel(dtype, head_dim, q_block, fusion, &fn, &threads)) return 0;
    int per_cu = 0, dev = -1, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return per_cu > 0 && cus > 0 ? per_cu * cus : 0;
}

int na_attn_launch(const NaAttnParams& p, int dtype, int head_dim, int q_block, bool fusion,
                   void* stream) {
    hipStream_t st = (hipStream_t)stream;
    // whole tiles, then the shares of the split tail tiles (none without a split)
    const dim3 grid((unsigned)(p.n_main + (int64_t)(p.n_wg - p.n_main) * p.n_split));
    const bool split = p.n_main < p.n_wg;
    const dim3 cgrid((unsigned)(((int64_t)(p.n_wg - p.n_main) * q_block * (head_dim / 4) + 255) / 256));
    const void* split_fn = nullptr;
    int split_threads = 0;
    if (split && (!split_kernel(dtype, head_dim, q_block, fusion, &split_fn, &split_threads) ||
                  p.sep_skip > 0))
        return (int)hipErrorInvalidValue;   // no shares with the bias or the fused partner branch
    if (fusion) {
        if (head_dim == 64 && q_block == 64)
            hipLaunchKernelGGL((attn_fwd_bf16<64, 2, true>), grid, dim3(128), 0, st, p);
        else if (head_dim == 64 && q_block == 128)
            hipLaunchKernelGGL((attn_fwd_bf16<64, 4, true>), grid, dim3(256), 0, st, p);
        else if (head_dim == 64 && q_block == 256)
            hipLaunchKernelGGL((attn_fwd_bf16<64, 8, true>), grid, dim3(512), 0, st, p);
        else if (head_dim == 128 && q_block == 128)
            hipLaunchKernelGGL((attn_fwd_bf16<128, 4, true>), grid, dim3(256), 0, st, p);
        else if (head_dim == 128 && q_block == 256)
            hipLaunchKernelGGL((attn_fwd_bf16<128, 8, true>), grid, dim3(512), 0, st, p);
        else
            return (int)hipErrorInvalidValue;
        return (int)hipGetLastError();
    }
    if (dtype == NA_BF16) {
        if (head_dim == 64 && q_block == 64) {
            hipLaunchKernelGGL((attn_fwd_bf16<64, 2>), grid, dim3(128), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<64, 64>), cgrid, dim3(256), 0, st, p);
        } else if (head_dim == 128 && q_block == 128) {
            hipLaunchKernelGGL((attn_fwd_bf16<128, 4>), grid, dim3(256), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<128, 128>), cgrid, dim3(256), 0, st, p);
        } else if (head_dim == 128 && q_block == 256) {
            hipLaunchKernelGGL((attn_fwd_bf16<128, 8>), grid, dim3(512), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<128, 256>), cgrid, dim3(256), 0, st, p);
        }
        else if (head_dim == 128 && q_block == 384) {
            hipLaunchKernelGGL((attn_fwd_bf16_m16<128, 8>), grid, dim3(512), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<128, 384>), cgrid, dim3(256), 0, st, p);
        }
        else if (head_dim == 64 && q_block == 128) {
            hipLaunchKernelGGL((attn_fwd_bf16<64, 4>), grid, dim3(256), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<64, 128>), cgrid, dim3(256), 0, st, p);
        } else if (head_dim == 64 && q_block == 256) {
            hipLaunchKernelGGL((attn_fwd_bf16<64, 8>), grid, dim3(512), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<64, 256>), cgrid, dim3(256), 0, st, p);
        }
        else if (head_dim == 128 && q_block == 192) {
            hipLaunchKernelGGL((attn_fwd_bf16_m16<128, 4>), grid, dim3(256), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<128, 192>), cgrid, dim3(256), 0, st, p);
        } else if (head_dim == 64 && q_block == 192) {
            hipLaunchKernelGGL((attn_fwd_bf16_m16<64, 4>), grid, dim3(256), 0, st, p);
            if (split) hipLaunchKernelGGL((attn_fwd_combine<64, 192>), cgrid, dim3(256), 0, st, p);
        }
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
