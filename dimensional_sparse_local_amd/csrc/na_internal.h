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
    na_plan_stats stats{};

    // device copies (null when host-only or not needed)
    bool on_device = false;
    int device = -1;
    int32_t* d_perm = nullptr;
    int32_t* d_row_ptr = nullptr;
    NaEntry* d_entries = nullptr;
    uint32_t* d_masks = nullptr;
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
};

// Returns false if no variant exists for (dtype, head_dim, q_block, kv_block).
bool na_attn_supported(int dtype, int head_dim, int q_block, int kv_block);
// Launch the fused attention kernel; returns the HIP error code (0 = success).
int na_attn_launch(const NaAttnParams& p, int dtype, int head_dim, int q_block, void* stream);

// Row gather / scatter (permute.hip): rows of row_bytes bytes (a multiple of 4);
// all strides in bytes.
int na_permute_launch(const void* in, void* out, int64_t B, int64_t H, int64_t N,
                      int64_t row_bytes, int64_t in_sb, int64_t in_sh, int64_t in_sn,
                      int64_t out_sb, int64_t out_sh, int64_t out_sn, const int32_t* perm,
                      int inverse, void* stream);
