// Device-side building blocks of libqkprep for gfx950 (CDNA4, wave64).
//
// - 16-byte vector loads and stores of bf16 head rows;
// - sums and maxima over the 8 or 16 lanes that hold one head row, built
//   from DPP lane permutes that never leave that lane group (the sum of
//   squares of an RMSNorm must cover one head of one token only: the review
//   of TensorRT-LLM's fused preprocessing kernel found a warp-wide sum that
//   mixed tokens);
// - bf16 and OCP FP8 E4M3 packing with the gfx950 conversion instructions
//   (v_cvt_pk_bf16_f32 rounds to nearest even; v_cvt_pk_fp8_f32 is used on
//   inputs clamped to +-448 first, which makes it round-to-nearest-even with
//   saturation, the "RN satfinite" of the FlashInfer contract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkprep {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// memory
// ---------------------------------------------------------------------------

// Loads through the global address space: a pointer chosen between two
// buffers (or built from a generic pointer) would otherwise be loaded with a
// flat instruction, whose wait also drains every outstanding load.
// (scalar and ext-vector types; the C-style cast is an address-space cast)
template <typename T>
__device__ __forceinline__ T gld(const T* p) {
    typedef const __attribute__((address_space(1))) T gT;
    return *(gT*)p;
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4_t v = gld(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming load (non-temporal hint): for data read exactly once, so that it
// does not displace what the caches hold for the writes in flight.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    typedef const __attribute__((address_space(1))) u32x4_t gT;
    const u32x4_t v = __builtin_nontemporal_load((gT*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st16(void* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// Streaming store (non-temporal hint): for data no kernel reads soon (the
// zeroed tail rows), so that it drains to memory during the kernel instead
// of staying dirty in the caches until the end-of-kernel write-back.
__device__ __forceinline__ void st16_stream(void* p, uint4 v) {
    typedef __attribute__((address_space(1))) u32x4_t gT;
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (gT*)p);
}

__device__ __forceinline__ void st8(void* p, uint2 v) {
    *reinterpret_cast<uint2*>(p) = v;
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void st8_stream(void* p, uint2 v) {
    typedef __attribute__((address_space(1))) u32x2_t gT;
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, (gT*)p);
}

// Row stores under the call's store policy: non-temporal (NT) for rows
// written to outputs no kernel of this call reads back, so that they drain
// to HBM as they are produced (with the previous calls' outputs still dirty
// in the caches, ordinary stores left the rows waiting in L2 and cost the
// 15k-token FP8 prefill about 8 % in steady state); ordinary stores when the
// caller keeps the rows in the caches for the next kernel, or when they are
// written back into lines the call has just read.
template <bool NT>
__device__ __forceinline__ void st16p(void* p, uint4 v) {
    if constexpr (NT) st16_stream(p, v);
    else st16(p, v);
}

template <bool NT>
__device__ __forceinline__ void st8p(void* p, uint2 v) {
    if constexpr (NT) st8_stream(p, v);
    else st8(p, v);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ldf4(const float* p) {
    const f32x4_t v = gld(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// Touch every dword of a kernel-argument struct at kernel entry.  The
// compiler otherwise loads each field from the kernarg segment where it is
// first used, and on a fresh launch each of those scalar loads misses: a
// kernel whose phases use different fields pays one memory round trip per
// phase.  Forcing all fields into SGPRs at entry turns that into one burst
// (for structs small enough to stay in SGPRs; the norm-rope-append kernel
// touches one dword per 32 bytes instead).
template <typename T>
__device__ __forceinline__ void preload_kernargs(const T& args) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&args);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(w[i]));
}

// n / d for 0 <= n < 2^31 with the host-computed multiplier of
// make_fastdiv31 (the sum below stays under 2^32)
struct FastDiv31;
template <typename FD>
__device__ __forceinline__ int fdiv31(int n, const FD& f) {
    const uint32_t t = __umulhi((uint32_t)n, f.m);
    return (int)((t + (uint32_t)n) >> f.l);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum of squares of the 8 bf16 values of a 16-byte vector, added to acc:
// v_dot2_f32_bf16 squares a packed bf16 pair (exact in fp32) and accumulates
// in fp32, so the unpacked values are not needed for it.
__device__ __forceinline__ float sumsq8_bf16(uint4 v, float acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t p = __builtin_bit_cast(bf16x2_t, w[i]);
        acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
    }
    return acc;
}

// 8 bf16 values of a 16-byte vector -> fp32 x[0..7]
__device__ __forceinline__ void unpack8(uint4 v, float* x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// two fp32 -> two bf16 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint4 pack8_bf16(const float* x) {
    uint4 r;
    r.x = pack_bf16x2(x[0], x[1]);
    r.y = pack_bf16x2(x[2], x[3]);
    r.z = pack_bf16x2(x[4], x[5]);
    r.w = pack_bf16x2(x[6], x[7]);
    return r;
}

// ---------------------------------------------------------------------------
// fp32 -> OCP E4M3, RN satfinite
// ---------------------------------------------------------------------------

__device__ __forceinline__ float sat448(float x) {
    return __builtin_fminf(__builtin_fmaxf(x, -kE4M3Max), kE4M3Max);
}

// four fp32 -> four E4M3 bytes, x0 in the lowest byte.  The conversion
// keeps the other half of its destination; the first one starts from x0's
// own bits (overwritten by the second), so no register has to be zeroed.
__device__ __forceinline__ uint32_t cvt_fp8x4(float x0, float x1, float x2, float x3) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_bit_cast(int, x0), false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, r, true);
    return (uint32_t)r;
}

__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
    return cvt_fp8x4(sat448(x0), sat448(x1), sat448(x2), sat448(x3));
}

// eight fp32 (multiplied by `scale`) -> eight E4M3 bytes
__device__ __forceinline__ uint2 pack8_fp8(const float* x, float scale) {
    uint2 r;
    r.x = pack_fp8x4(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
    r.y = pack_fp8x4(x[4] * scale, x[5] * scale, x[6] * scale, x[7] * scale);
    return r;
}

// The same without the saturation, for a scale derived from the values'
// own amax: then |x * scale| <= upper_max (1 + a few ulp) <= 448.0002, which
// the conversion already rounds to 448 (it returns NaN only above 464).
__device__ __forceinline__ uint2 pack8_fp8_bounded(const float* x, float scale) {
    uint2 r;
    r.x = cvt_fp8x4(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
    r.y = cvt_fp8x4(x[4] * scale, x[5] * scale, x[6] * scale, x[7] * scale);
    return r;
}

// ---------------------------------------------------------------------------
// lane-group reductions (G = 8 or 16 lanes, aligned to multiples of G)
// ---------------------------------------------------------------------------

// DPP controls (gfx9 encoding)
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float,
        __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the G consecutive lanes of a lane group; every lane of the
// group receives the total.  All lanes of the group must be active.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 4 || G == 8 || G == 16, "lane groups of 4, 8 or 16");
    v += dpp_f<kDppQuadSwap1>(v);
    v += dpp_f<kDppQuadSwap2>(v);
    if constexpr (G >= 8) v += dpp_f<kDppRowHalfMirror>(v);  // lane i <- lane 7 - i (other quad of the 8)
    if constexpr (G == 16) v += dpp_f<kDppRowMirror>(v);     // lane i <- lane 15 - i
    return v;
}

// Max of non-negative floats (amax values) over a lane group.  For
// non-negative floats the order of the values is the order of their bit
// patterns, so the reduction runs on unsigned integers: a float max of a
// value moved by DPP would first be canonicalised, one more instruction
// per step.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
    static_assert(G == 4 || G == 8 || G == 16, "lane groups of 4, 8 or 16");
    uint32_t u = __float_as_uint(v);
    u = max(u, dpp_u<kDppQuadSwap1>(u));
    u = max(u, dpp_u<kDppQuadSwap2>(u));
    if constexpr (G >= 8) u = max(u, dpp_u<kDppRowHalfMirror>(u));
    if constexpr (G == 16) u = max(u, dpp_u<kDppRowMirror>(u));
    return __uint_as_float(u);
}

// max(a, b) of non-negative floats, as above
__device__ __forceinline__ float max_nonneg(float a, float b) {
    return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
}

// Whole-line loads for lanes that do not own the whole line.  When four
// lanes hold a 128-byte row as two 16-byte vectors each, a load instruction
// in which every lane reads its own vector covers only half of each row's
// line.  Rows are then loaded in pairs, one whole line per instruction, and
// this exchange completes them.  Each lane loaded v0 and v1; a DPP mirror
// (CTRL) pairs it with a partner,
// and lanes in the banks of RECV_FIRST take the partner's v1 as their first
// vector, lanes in the banks of RECV_SECOND the partner's v0 as their second
// (DPP banks are the 4-lane groups of each 16-lane row).
//  - Four lanes per 128-byte row (row_half_mirror, 0xA / 0x5): lanes
//    8p .. 8p+3 (row 2p) loaded v0 = their own first vector and v1 = the
//    first vector of their mirror partner in row 2p+1; lanes 8p+4 .. 8p+7
//    (row 2p+1) loaded v0 = their partner's second vector in row 2p and v1 =
//    their own second vector.  In the whole-head layout (elements [8 gl, +8)
//    and [32 + 8 gl, +8) per lane) that is row 2p [8 gl, +8) and row 2p+1
//    [24 - 8 gl, +8) for lane gl of row 2p, row 2p [56 - 8k, +8) and row 2p+1
//    [32 + 8k, +8) for lane k of row 2p+1.
//  - Rotary over half the head, 8 or 16 lanes per row (row_half_mirror 0xA /
//    0x5, or row_mirror 0xC / 0x3): rope lane gl (< G/2) loaded v0 = [8 gl,
//    +8) and v1 = the first vector [16 (G-1-gl), +8) of pass lane G-1-gl; pass
//    lane gl loaded v0 = the second vector [R/2 + 8 (G-1-gl), +8) of rope lane
//    G-1-gl and v1 = its own [16 gl + 8, +8).
template <int CTRL, int RECV_FIRST, int RECV_SECOND>
__device__ __forceinline__ void mirror_exchange(uint4& v0, uint4& v1) {
    uint4 f, g;
    f.x = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.x, (int)v1.x, CTRL, 0xF, RECV_FIRST, false);
    f.y = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.y, (int)v1.y, CTRL, 0xF, RECV_FIRST, false);
    f.z = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.z, (int)v1.z, CTRL, 0xF, RECV_FIRST, false);
    f.w = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.w, (int)v1.w, CTRL, 0xF, RECV_FIRST, false);
    g.x = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.x, (int)v0.x, CTRL, 0xF, RECV_SECOND, false);
    g.y = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.y, (int)v0.y, CTRL, 0xF, RECV_SECOND, false);
    g.z = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.z, (int)v0.z, CTRL, 0xF, RECV_SECOND, false);
    g.w = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.w, (int)v0.w, CTRL, 0xF, RECV_SECOND, false);
    v0 = f;
    v1 = g;
}

// The same exchange for rotary over more than half the head: with P
// pass-through lanes per row, only the P lowest lanes (rope lanes that loaded
// their mirror partner's first vector as v1) and the P highest (pass lanes
// that loaded their partner's second vector as v0) trade; the rope lanes in
// between loaded both of their own vectors.  Every lane takes the mirrored
// value and keeps it only where it receives.
template <int CTRL>
__device__ __forceinline__ void mirror_exchange_sel(uint4& v0, uint4& v1, bool recv_first, bool recv_second) {
    uint4 f, g;
    f.x = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.x, (int)v1.x, CTRL, 0xF, 0xF, false);
    f.y = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.y, (int)v1.y, CTRL, 0xF, 0xF, false);
    f.z = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.z, (int)v1.z, CTRL, 0xF, 0xF, false);
    f.w = (uint32_t)__builtin_amdgcn_update_dpp((int)v0.w, (int)v1.w, CTRL, 0xF, 0xF, false);
    g.x = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.x, (int)v0.x, CTRL, 0xF, 0xF, false);
    g.y = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.y, (int)v0.y, CTRL, 0xF, 0xF, false);
    g.z = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.z, (int)v0.z, CTRL, 0xF, 0xF, false);
    g.w = (uint32_t)__builtin_amdgcn_update_dpp((int)v1.w, (int)v0.w, CTRL, 0xF, 0xF, false);
    if (recv_first) v0 = f;
    if (recv_second) v1 = g;
}

// ---------------------------------------------------------------------------
// wave and block primitives
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave with DPP: Hillis-Steele
// inside each row of 16 lanes (row_shr 1, 2, 4, 8), then the row totals are
// carried across rows with row_bcast:15 (into rows 1 and 3) and row_bcast:31
// (into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// OR of `v` over the workgroup (4 waves) with a single barrier; `slot` is
// 4 ints of LDS used by this call site only.
__device__ __forceinline__ int block_or4(int v, int* slot) {
    const bool any = __ballot(v != 0) != 0;
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = any ? 1 : 0;
    __syncthreads();
    return slot[0] | slot[1] | slot[2] | slot[3];
}

// ---------------------------------------------------------------------------
// one 16-byte store per lane for an FP8 head row
// ---------------------------------------------------------------------------

// Lane gl of a head-row group holds the E4M3 codes of dims [8 gl, 8 gl + 8)
// (lo) and [half + 8 gl, half + 8 gl + 8) (hi).  Neighbouring lanes swap one
// 8-byte half so that even lanes store dims [8 gl, 8 gl + 16) and odd lanes
// dims [half + 8 gl - 8, half + 8 gl + 8): one 16-byte store per lane, and
// the group writes whole 128-byte lines.
template <bool NT>
__device__ __forceinline__ void store_fp8_row(uint8_t* row, int gl, int half, uint2 lo, uint2 hi) {
    const bool odd = gl & 1;
    const uint2 send = odd ? lo : hi;
    uint2 recv;
    recv.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.x, kDppQuadSwap1, 0xF, 0xF, false);
    recv.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.y, kDppQuadSwap1, 0xF, 0xF, false);
    const uint4 v = odd ? make_uint4(recv.x, recv.y, hi.x, hi.y) : make_uint4(lo.x, lo.y, recv.x, recv.y);
    st16p<NT>(row + (odd ? half + 8 * (gl - 1) : 8 * gl), v);
}

}  // namespace qkprep
