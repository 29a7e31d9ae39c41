// Launch descriptors shared by the C-ABI layer and the kernels of libqkprep.
// Host-validated copies of the public params, flattened to what the device
// needs, plus the launch geometry chosen on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkprep {

// Largest batch the norm-rope-append kernel stages in LDS (q_indptr,
// seq_lens and a page-count prefix: 12 bytes per request).
constexpr int kMaxRequests = 4096;
constexpr int kBlockThreads = 256;
constexpr int kMaxTokensPerTile = 16;
// largest Hq whose per-tile padded Q scales are gathered in LDS
constexpr int kMaxStagedQHeads = 256;
// head rows each wave has in flight per load batch (double-buffered)
constexpr int kBatch = 2;
// tail pages of the first requests a workgroup clears, prefetched with the metadata
constexpr int kTailPrefetch = 16;
// XCDs of the part (workgroups are dealt to them round-robin by index) and
// the number of consecutive round-robin spans of a long call kept on one XCD
constexpr int kXcds = 8;
constexpr int kXcdRun = 16;
// decodes with at least this many requests clear the tails after the token rows
constexpr int kTailsLastRequests = 256;
// workgroups that share the tail clears of a call with fewer requests
// (one per CU of the 256 CUs of the part)
constexpr int kTailSpreadGroups = 256;
// up to this many requests the validation finds a page's request by binary
// search, and reads the page ids as 16-byte vectors when the table allows it
constexpr int kSearchRequests = 64;

// Division of a non-negative 31-bit integer by a runtime divisor d >= 1
// without a division instruction (Granlund and Montgomery, "Division by
// invariant integers using multiplication", round-up variant):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv31 {
    uint32_t m;
    uint32_t l;
    uint32_t d;
};

inline FastDiv31 make_fastdiv31(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv31 f;
    f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    f.l = l;
    f.d = d;
    return f;
}

// Memory modes of the norm-rope-append kernel: Q or K written back into
// qkv (cached loads and stores); qkv read once with streaming loads, and the
// Q rows stored with streaming (non-temporal) or ordinary stores (K/V cache
// rows always take ordinary stores).
enum : int { kMemInPlace = 0, kMemStream = 1, kMemKeep = 2 };

struct NraDevArgs {
    // shapes
    int32_t T, Hq, Hkv, R;             // R = Hq + 2 Hkv head rows per token
    const uint16_t* qkv;
    int64_t qkv_stride;
    int32_t norm;                       // 0 none, 1 rms, 2 gemma
    float eps;
    const float* q_w;
    const float* k_w;
    int32_t rope;                       // 0 neox, 1 interleaved
    int32_t rot;                        // rotated dims per head: 0..D, multiple of 16
    const float* cos_sin;               // [cs_rows, rot]
    int64_t cs_rows;
    const int64_t* positions;
    int32_t paged;                      // 1 page table, 0 slot mapping
    int32_t B;
    const int32_t* q_indptr;
    const int32_t* seq_lens;
    const int32_t* page_table;
    int32_t maxp;
    const int64_t* slot_mapping;
    void* k_cache;
    void* v_cache;
    int32_t num_pages, page_size;
    FastDiv31 ps_div;                   // division by page_size
    int64_t k_page_stride, v_page_stride;
    const float* k_scale;
    const float* v_scale;
    int32_t zero_tail;
    void* q_out;
    int64_t q_out_stride;
    float* q_scale;
    int32_t q_scale_padded;
    int32_t max_seqlen;
    int64_t q_scale_P;                  // padded row length round_up(max_seqlen, 128)
    int32_t stage_q_scale;              // gather padded scales per tile in LDS
    const float* q_scale_inv;
    float upper_max;
    uint16_t* k_out;
    int64_t k_out_stride;
    int32_t* flags;
    // geometry: every workgroup owns a balanced, contiguous range of the
    // T * chunks_per_token (token, chunk) items and of the B requests
    int32_t tokens_per_tile;            // most tokens staged in LDS at once
    int32_t chunks_per_token;           // ceil(R / head rows per wave)
    int64_t total_items;                // T * chunks_per_token
    // K/V redirect: k_cache / v_cache point at out_k / out_v, rows by token
    int32_t redirect;
    int64_t kv_out_stride;              // elements between token rows (redirect)
    // dynamic FP8 K/V scales: dims per scale (0 = static scalars)
    int32_t kv_group;
    float* k_scale_out;
    float* v_scale_out;
    int32_t mem;                        // kMemInPlace / kMemStream / kMemKeep
    int32_t pt_vec;                     // page ids read as 16-byte vectors: B <= kSearchRequests, table
                                        // 16-byte aligned, maxp a multiple of 4, paged, not redirected
    int32_t interleave;                 // items per round-robin span, 0 = one range per workgroup
    int32_t grid;                       // workgroups launched (set by the launcher)
    // divisions of the launch geometry without a division instruction (set
    // by the launcher): by grid, by chunks_per_token, by B (1 when B = 0),
    // and total_items = items_q * grid + items_r
    FastDiv31 grid_div, cpt_div, b_div;
    int32_t items_q, items_r;
};

struct MlaDevArgs {
    int32_t T, H, nope_dim, kv_lora_rank;
    uint16_t* q;
    int64_t q_token_stride, q_head_stride;
    const uint16_t* kv_c;
    int64_t kv_c_stride;
    const uint16_t* k_pe;
    int64_t k_pe_stride;
    int32_t rope;
    const float* cos_sin;
    int64_t cs_rows;
    const int64_t* positions;
    const int64_t* slot_mapping;
    void* kv_cache;
    int64_t capacity;                   // num_blocks * block_size
    int32_t block_size;
    int64_t block_stride;
    const float* kv_scale;
    // FP8 Q output (q_mode 1 dynamic per token, 2 static)
    int32_t q_mode;
    uint8_t* q_out;
    int64_t q_out_token_stride, q_out_head_stride;
    float* q_scale;
    const float* q_scale_inv;
    float upper_max;
    int32_t nt_store;                   // 1: streaming (non-temporal) row stores
    // geometry: balanced contiguous ranges of the T * chunks_per_token items
    int32_t tokens_per_tile;            // most tokens staged in LDS at once
    int32_t chunks_per_token;           // ceil(H / heads per wave) + 1 latent chunk
    int64_t total_items;
    int32_t grid;                       // workgroups launched (set by the launcher)
    // divisions without a division instruction (set by the launcher): by
    // grid, by chunks_per_token, by block_size (used when capacity < 2^31),
    // and total_items = items_q * grid + items_r
    FastDiv31 grid_div, cpt_div, bs_div;
    int32_t items_q, items_r;
};

// Workgroups of kBlockThreads threads that `kernel` keeps resident on the
// current device with `dyn_lds` bytes of dynamic LDS, over all CUs.  Queried
// once per (kernel, device, dyn_lds) and cached; safe to call from several
// host threads.  Returns 0 if the device cannot be queried (a failed query's
// error is cleared, so that it is not taken for a launch error).
int resident_grid(const void* kernel, size_t dyn_lds);

// returns hipSuccess or the launch error
// one object of nra_kernel.hip per head dim
hipError_t launch_norm_rope_append_d64(const NraDevArgs& a, int q_mode, int kv_fp8, hipStream_t stream);
hipError_t launch_norm_rope_append_d128(const NraDevArgs& a, int q_mode, int kv_fp8, hipStream_t stream);
hipError_t launch_norm_rope_append_d256(const NraDevArgs& a, int q_mode, int kv_fp8, hipStream_t stream);

inline hipError_t launch_norm_rope_append(const NraDevArgs& a, int head_dim, int q_mode, int kv_fp8,
                                          hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_norm_rope_append_d64(a, q_mode, kv_fp8, stream);
        case 128: return launch_norm_rope_append_d128(a, q_mode, kv_fp8, stream);
        case 256: return launch_norm_rope_append_d256(a, q_mode, kv_fp8, stream);
        default: return hipErrorInvalidValue;
    }
}
hipError_t launch_mla_concat_rope(const MlaDevArgs& a, int kv_fp8, hipStream_t stream);
// FP8 Q modes: one workgroup per token at a time
hipError_t launch_mla_q8(const MlaDevArgs& a, int kv_fp8, hipStream_t stream);

}  // namespace qkprep
