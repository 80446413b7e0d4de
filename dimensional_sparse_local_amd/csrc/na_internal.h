// Internal declarations shared by the planner, the ABI glue and the kernel
// launchers of libna.so.  Not part of the public ABI (include/na.h is).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "na.h"

// Query / key-value tile lengths of the bf16 and fp32 kernels.
constexpr int NA_KV_BLOCK_BF16 = 64;
constexpr int NA_KV_BLOCK_F32 = 32;
constexpr int NA_Q_BLOCK_F32 = 32;

// One non-empty (query tile, key/value tile) pair of a CSR row: the key/value
// tile and the index of the bit mask to apply, or -1 when every (valid query,
// key) pair of the two tiles is attended and no key lies past the last token.
struct NaEntry {
    int32_t kt;
    int32_t mask;
};

// One query tile of the paired key-major map (gradients of K and V): the
// query tile and the mask ids for the two key/value tiles of the pair
// (-1 = every pair attended, -2 = the query tile does not attend that tile).
struct NaPairEntry {
    int32_t qt;
    int32_t mask0;
    int32_t mask1;
    int32_t pad;
};
constexpr int32_t NA_MASK_NONE = -2;

struct na_plan_s {
    na_plan_desc desc;        // normalised copy (defaults filled in)
    int64_t n_tokens = 0;
    int32_t pdims = 0;        // pattern dimensions (ndim, or 1 for Hilbert)
    int32_t plen[3] = {1, 1, 1};
    int32_t left[3] = {0, 0, 0};
    int32_t clamp[3] = {1, 1, 1};
    bool identity_order = true;
    bool has_dilation = false;
    std::vector<int32_t> perm;      // sequence position -> row-major token
    std::vector<int32_t> row_ptr;   // n_q_tiles + 1
    std::vector<NaEntry> entries;   // CSR column: non-empty key/value tiles
    std::vector<uint8_t> entry_cls; // 1 partial, 2 full (per entry)
    std::vector<int32_t> kcoord;    // [N][4]: pattern coordinates of each position
    std::vector<int32_t> qbox;      // [N][8]: lo[3], hi[3] of each position's window
    // Deduplicated tile masks: mask m, query row r of its tile, word w holds
    // keys 32w .. 32w+31 of the key/value tile (bit set = attended).
    int32_t mask_words = 0;         // ceil(kv_block / 32)
    std::vector<uint32_t> masks;    // [n_masks][q_block][mask_words]
    int64_t n_masks = 0;
    // pi-Attention partner: partner_union = the partners are part of the tile
    // map (union and fixed-fusion modes); with fixed fusion, skip_masks (same
    // layout and ids as masks) marks the partners outside the window, whose
    // logits carry the extra log((1 - alpha) / alpha).
    bool partner_union = false;
    std::vector<uint32_t> skip_masks;
    // The same tile map by key/value tile (for the gradients of K and V): for
    // key/value tile kt, entries t_row_ptr[kt] .. t_row_ptr[kt+1] of t_entries
    // hold the query tiles that attend it (field kt = query tile) in ascending
    // order, with the mask ids of the query-major map.
    std::vector<int32_t> t_row_ptr; // n_kv_tiles + 1
    std::vector<NaEntry> t_entries;
    // The same by pairs of key/value tiles (2g, 2g + 1): the union of their
    // query tiles in ascending order, with both mask ids.
    std::vector<int32_t> p_row_ptr; // ceil(n_kv_tiles / 2) + 1
    std::vector<NaPairEntry> p_entries;
    na_plan_stats stats{};
    int32_t max_row_len = 0;        // most non-empty key/value tiles of one query tile
    // workgroups of this plan's forward kernel that fit on the device at once
    // (compute units x workgroups per unit), for kernels with a split-walk
    // mode; 0 otherwise or for host-only plans
    int32_t split_capacity = 0;
    // dispatch the query tiles of each (batch, head) in descending order: set
    // for one-dimensional maps whose walks grow along the sequence (causal
    // windows), so that the short walks at its start come last
    bool q_desc = false;

    // device copies (null when host-only or not needed)
    bool on_device = false;
    int device = -1;
    int32_t* d_perm = nullptr;
    int32_t* d_row_ptr = nullptr;
    NaEntry* d_entries = nullptr;
    uint32_t* d_masks = nullptr;
    uint32_t* d_skip_masks = nullptr;
    int32_t* d_t_row_ptr = nullptr;
    NaEntry* d_t_entries = nullptr;
    int32_t* d_p_row_ptr = nullptr;
    NaPairEntry* d_p_entries = nullptr;
    void* d_zero = nullptr;   // 1 KiB of zeros
};

// Thread-local error detail.
void na_set_error(const char* fmt, ...);

// Host planner (plan.cpp).
na_status na_plan_build_host(const na_plan_desc* desc, na_plan_s* plan);

// Kernel launch parameters (attn_fwd.hip).
struct NaAttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int32_t n_tokens;
    int32_t heads;
    int32_t n_q_tiles;
    int32_t n_wg;          // n_q_tiles * B * H
    float scale_log2;      // scale * log2(e)
    const int32_t* perm;   // null = identity addressing
    const int32_t* row_ptr;
    const NaEntry* entries;
    const uint32_t* masks;  // [n_masks][q_block][mask_words]
    const void* zero;       // >= 1 KiB of zeros: the source of rows past the last token
    // fixed fusion only (else null / 0): partner bit planes, the bias added to
    // the raw dot product q.k of a partner (log((1 - alpha) / alpha) / scale)
    // and the shift added to lse (log alpha)
    const uint32_t* skip_masks;
    float skip_bias;
    float lse_shift;
    // separate-softmax partner branch fused into the epilogue of the bf16
    // kernels with 32 queries per wave (0 = none): the partner distance on the
    // sequence and whether x + pi is fetched too
    int32_t sep_skip;
    int32_t sep_both;
    // split tail (48-query-per-wave kernels): workgroups below n_main run
    // whole query tiles (index remapped over n_main); the rest run part
    // (index - n_main) % n_split of tile n_main + (index - n_main) / n_split:
    // that share of its walk, writing unnormalised partial results to part_o
    // ([part][q_block][head_dim] fp32) and part_ml ([part][q_block][2]: the
    // row's reference maximum (log2 domain) and its row sum), which
    // attn_fwd_combine merges.  n_main = n_wg and n_split = 1 for no split.
    int32_t n_main;
    int32_t n_split;
    float* part_o;
    float* part_ml;
    // 1: query tiles of each (batch, head) in descending order (tile_of)
    int32_t q_desc;
};

// Gradient launch parameters (attn_bwd.hip).  Tensors as in NaAttnParams;
// g = dout, lse and delta are fp32 [B][H][N] in row-major token order.
struct NaBwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    float* delta;          // workspace: dout_i . out_i
    void* dq;
    void* dk;
    void* dv;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int64_t g_sb, g_sh, g_sn;
    int64_t dq_sb, dq_sh, dq_sn;
    int64_t dk_sb, dk_sh, dk_sn;
    int64_t dv_sb, dv_sh, dv_sn;
    int32_t batch;
    int32_t n_tokens;
    int32_t heads;
    int32_t n_q_tiles;
    int32_t n_kv_tiles;
    int32_t q_block;
    float scale;
    float scale_log2;      // scale * log2(e)
    const int32_t* perm;   // null = identity addressing
    const int32_t* row_ptr;
    const NaEntry* entries;
    const int32_t* t_row_ptr;
    const NaEntry* t_entries;
    const int32_t* p_row_ptr;     // paired key-major map
    const NaPairEntry* p_entries;
    const uint32_t* masks;
    const void* zero;      // >= 1 KiB of zeros
    // fixed fusion only (as in NaAttnParams): partner planes, the partners'
    // raw dot-product bias and the log(alpha) the forward added to lse
    const uint32_t* skip_masks;
    float skip_bias;
    float lse_shift;
    // separate-softmax partners (pi_skip.hip): x - skip (and x + skip)
    int32_t skip;
    int32_t skip_both;
};

// Returns false if no gradient kernels exist for (dtype, head_dim, q_block, kv_block).
bool na_bwd_supported(int dtype, int head_dim, int q_block, int kv_block);
// Launch the three gradient kernels (row sums, dq, dk/dv); HIP error code.
// fusion = the fixed-fusion (logit bias) variants; with_delta = false skips the
// row sums (the caller has written p.delta).
int na_bwd_launch(const NaBwdParams& p, int head_dim, bool fusion, bool with_delta, void* stream);
// Device address and size of this GPU's fixed delta scratch (attn_bwd.hip),
// looked up once per device; 0 or a hipError_t.
int na_bwd_scratch(void** ptr, size_t* bytes);

// Returns false if no variant exists for (dtype, head_dim, q_block, kv_block);
// fusion = the fixed-fusion (logit bias) variant.
bool na_attn_supported(int dtype, int head_dim, int q_block, int kv_block, bool fusion);
// Launch the fused attention kernel; returns the HIP error code (0 = success).
// Workgroups of the forward kernel for (dtype, head_dim, q_block, fusion)
// resident on the current device at once, if that kernel has the split-walk
// mode; 0 otherwise.
int na_attn_split_capacity(int dtype, int head_dim, int q_block, bool fusion);
int na_attn_launch(const NaAttnParams& p, int dtype, int head_dim, int q_block, bool fusion,
                   void* stream);

// The partner branch of the separate-softmax variant (pi_skip.hip): for every
// query, out += softmax over its partners of z, applied to their v rows.
struct NaSkipParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int32_t batch;
    int32_t heads;
    int32_t n_tokens;
    int32_t skip;
    int32_t skip_both;
    float scale;
    const int32_t* perm;   // null = identity addressing
};
bool na_skip_supported(int dtype, int head_dim);
int na_skip_launch(const NaSkipParams& p, int dtype, int head_dim, void* stream);
// Gradients of the separate-softmax variant (bf16): delta_i of the window
// branch alone (before the gradient kernels, in place of their row sums), and
// the partner branch's dq, dk, dv added to theirs (after).
int na_skip_bwd_delta_launch(const NaBwdParams& p, int head_dim, void* stream);
int na_skip_bwd_grads_launch(const NaBwdParams& p, int head_dim, void* stream);

// Row gather / scatter (permute.hip): rows of row_bytes bytes (a multiple of 4);
// all strides in bytes.
int na_permute_launch(const void* in, void* out, int64_t B, int64_t H, int64_t N,
                      int64_t row_bytes, int64_t in_sb, int64_t in_sh, int64_t in_sn,
                      int64_t out_sb, int64_t out_sh, int64_t out_sn, const int32_t* perm,
                      int inverse, void* stream);
