// Shared by the chunked prefill kernels (bf16 and fp32 inputs): the kernel
// parameter block, the sequence lookup and small device helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {
namespace pf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kC = 64;        // chunk length
constexpr int kScRows = 5;    // per-token scale rows in the workspace

// Rows of the per-(chunk, head) scale block.
enum : int {
    kScX = 0,     // exp(gamma_r) rk_r            scales X = K H
    kScBeta = 1,  // beta_r
    kScZ = 2,     // exp(gamma_r) rq_r            scales Z = Q H
    kScD = 3,     // rk_r exp(gamma_last - gamma_r)  scales U in the state advance
    kScE = 4,     // exp(gamma_last)              (every entry)
};

// fp32 T and P in the workspace: the ten 16 x 16 blocks (tau, j), j <= tau,
// of the lower triangle of a 64 x 64 matrix, block (tau, j) at index
// tau (tau + 1) / 2 + j, each as 64 lanes x 4 floats with lane (row, g)
// holding X[16 tau + row][16 j + 4 g + e].
constexpr int kFragFloats = 10 * 64 * 4;

constexpr int kInlineSeqs = 32;

struct PrefillParams {
    const int32_t* cu;          // [N+1] device
    const int32_t* chunk_off;   // [N+1] device (workspace): first chunk of each sequence
    const uint16_t* q;          // [T][HK][DK] bf16 bits
    const uint16_t* k;
    const uint16_t* v;          // [T][HV][DV]
    const float* g;             // [T][HV]
    const float* beta;
    uint16_t* o;                // [T][HV][DV]
    float* pool;
    const int32_t* src;
    const int32_t* dst;
    int32_t* err;
    // the same arrays when the inputs are float32
    const float* qf;
    const float* kf;
    const float* vf;
    float* of;
    float* tpf;                 // [chunks][HV][2][10][64][4] T, then P, as fp32 row fragments
    const int32_t* ckpt;        // [chunks] device or null: slot receiving the state after each chunk
    uint16_t* tp;               // [chunks][HV][2][64 * 64] T, then P, as row-operand fragments
    float* sc;                  // [chunks][HV][5][64]    scale rows
    int32_t* chunk_off_w;       // same buffer as chunk_off, written by the prep kernel
    const int32_t* seg_off;     // [N+1] device (workspace): first segment of each sequence
    int32_t* seg_off_w;
    float* se;                  // [segs][HV][DK][DV]   local end state E of each segment (split only)
    uint16_t* sm;               // [segs][HV][2][DK][DK] transition M, bf16 high and low parts (split only)
    float* sh;                  // [segs][HV][DK][DV]   copy of the initial state at a split sequence's first segment
    int32_t seg_len;            // chunks per segment; 0 = one segment per sequence
    int32_t num_segs;
    int32_t n_seqs;
    int32_t num_chunks;
    int32_t total_tokens;
    int32_t hk;
    int32_t hv;
    int32_t group;
    int32_t dkq;                // dk of q, k and the pool tiles; the kernels run at DK >= dkq
                                // (dk = 16 runs at DK = 32 with zero-padded rows and columns)
    int32_t dv;
    int32_t num_slots;
    float scale;
    float eps;
    // For calls of at most kInlineSeqs sequences the host fills both offset
    // tables here (the kernel arguments) and the prep kernel is not launched;
    // inl_n is then n_seqs, else 0.
    int32_t inl_n;
    int32_t inl_chunk[kInlineSeqs + 1];
    int32_t inl_seg[kInlineSeqs + 1];
};

// Chunk range [c0, c1) and segment range [s0, s1) of sequence n.
struct SeqSpan {
    int n, c0, c1, s0, s1;
};

// The span of the sequence holding chunk `key` (BY_SEG false) or segment
// `key` (BY_SEG true): the last sequence whose first chunk (segment) is
// <= key. `key` is wave-uniform. The kernel-argument tables are only ever
// indexed by constants (a fully unrolled scan), so they stay in the argument
// segment instead of being copied to private memory.
template <bool BY_SEG>
__device__ __forceinline__ SeqSpan find_span(const PrefillParams& p, int key) {
    SeqSpan r;
    if (p.inl_n > 0) {
        r = SeqSpan{0, p.inl_chunk[0], p.inl_chunk[1], p.inl_seg[0], p.inl_seg[1]};
        if (p.inl_n == 1) return r;
#pragma unroll
        for (int i = 1; i < kInlineSeqs; ++i) {
            if (i < p.inl_n && (BY_SEG ? p.inl_seg[i] : p.inl_chunk[i]) <= key)
                r = SeqSpan{i, p.inl_chunk[i], p.inl_chunk[i + 1], p.inl_seg[i], p.inl_seg[i + 1]};
        }
        return r;
    }
    const int32_t* off = BY_SEG ? p.seg_off : p.chunk_off;
    int lo = 0, hi = p.n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= key) lo = mid;
        else hi = mid - 1;
    }
    return SeqSpan{lo, p.chunk_off[lo], p.chunk_off[lo + 1], p.seg_off[lo], p.seg_off[lo + 1]};
}

// Buffer resources (base, byte range): loads past the range return zero and
// stores past it are dropped, in hardware, so ragged rows need no branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, 0, 0);
}
__device__ __forceinline__ f32x4 buf_load_f4(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f1(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store_f1(float v, rsrc_t r, unsigned off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0)), v),
                                          r, off, 0, 0);
}

// 2^x on the hardware exp2 (v_exp_f32). Arguments here are <= 0 decay
// exponents; results below the normal range flush to zero, which is the
// decay factor's limit anyway.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only. A plain __syncthreads() also waits
// for every outstanding global load and store of the wave (the workgroup
// release fence covers global memory), which would put a full memory round
// trip on every chunk; the kernels here exchange data between waves through
// LDS alone.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// fp32 16 x 16 x 16 product on the fp32 MFMA: acc += X Y, with X given with
// one row per lane (lane (row, g) holds X[row][4 g + e]) and Y in accumulator
// layout (lane (column, g) holds Y[4 g + e][column]). Step kk contracts
// k = 4 g + kk, so both operands are read in place. Swapping the arguments
// yields (X Y)^T in accumulator layout, i.e. X Y with one row per lane.
__device__ __forceinline__ f32x4 mm16(f32x4 x, f32x4 y, f32x4 acc) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[kk], y[kk], acc, 0, 0, 0);
    return acc;
}

// The fp32 recurrence across chunks (float32 inputs), after the fp32
// intra-chunk kernel has filled T, P and the scale rows.
int launch_f32_recurrence(const PrefillParams& p, hipStream_t s);

}  // namespace pf
}  // namespace gdn
