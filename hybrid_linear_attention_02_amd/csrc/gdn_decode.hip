// Single-token decode of the gated delta rule over a slot pool (gfx950).
//
// Per (request b, value head h) the update reads the source tile H = S^T
// (dk x dv float32) once and writes the destination tile once:
//
//   a = H^T k^,  c = H^T q~                       (reductions over dk)
//   u = beta (v - exp(g) a)                       (delta-rule correction)
//   o = exp(g) c + u (k^ . q~)                    (read-out on the new state)
//   H' = exp(g) H + k^ u^T                        (decay + rank-one write)
//
// which is the rule S <- exp(g) S; S <- S + beta (v - S k^) k^T; o = S q~ with
// the read-out expanded so that the tile is streamed in a single pass.
// Source/destination slots come from index tables, so a cached checkpoint is
// read and never written, and advancing a request moves no state bytes -- the
// index indirection of the TokenSpeed article (24-ai.news, English), section
// "What are the key optimizations behind the record?", item "Mamba State
// Update optimization".
//
// The work is bound by HBM bandwidth (about 0.9 flop per byte), so the kernel
// uses no matrix cores: each thread owns float4 column groups of several rows,
// loads them with 128-bit non-temporal loads (the tile is touched once), keeps
// them in registers across the reduction, reduces over dk with cross-lane
// shuffles and one small LDS exchange between waves, and writes the new tile
// with 128-bit non-temporal stores.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gdn_internal.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    void* o;
    float* pool;
    const int32_t* src;
    const int32_t* dst;
    int32_t* err;
    int32_t hk;
    int32_t hv;
    int32_t group;      // hv / hk
    int32_t num_slots;
    float scale;
    float eps;
    int32_t ndraft;           // verify: draft tokens per request (K); decode: 1
    const int32_t* lens;      // verify: [B] draft lengths or null (all K)
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element access for the two input types; bf16 is carried as uint16 bits.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static __device__ __forceinline__ float load(const void* p, size_t i) { return static_cast<const float*>(p)[i]; }
    static __device__ __forceinline__ f4 load4(const void* p, size_t i) {
        return *reinterpret_cast<const f4*>(static_cast<const float*>(p) + i);
    }
    static __device__ __forceinline__ void store4(void* p, size_t i, f4 x) {
        *reinterpret_cast<f4*>(static_cast<float*>(p) + i) = x;
    }
};

template <>
struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const void* p, size_t i) {
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    static __device__ __forceinline__ f4 load4(const void* p, size_t i) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        f4 r;
        r.x = __uint_as_float(w.x << 16);
        r.y = __uint_as_float(w.x & 0xffff0000u);
        r.z = __uint_as_float(w.y << 16);
        r.w = __uint_as_float(w.y & 0xffff0000u);
        return r;
    }
    static __device__ __forceinline__ void store4(void* p, size_t i, f4 x) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
    }
};

// Thread layout of one (request, head) tile: CG float4 column groups per row,
// RG row groups; thread t owns column group t % CG of rows t / CG + RG * m.
constexpr int decode_threads(int dk, int dv) { return (dk * dv / 4 < 256) ? dk * dv / 4 : 256; }

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NT = decode_threads(DK, DV);  // threads, a multiple of 64
    static constexpr int CG = DV / 4;
    static constexpr int RG = NT / CG;
    static constexpr int RPT = DK / RG;   // rows per thread
    static constexpr int NW = NT / 64;    // waves
    static_assert(NT % 64 == 0 && 64 % CG == 0 && DK % RG == 0, "unsupported tile shape");
};

// LDS of one (request, head) workgroup: each wave's own copy of k^ and q~
// (written and read by that wave alone), and the waves' partial reductions
// in two sets, so that consecutive tokens of a verify chain alternate.
template <int DK, int DV>
struct TokenScratch {
    float k[DecodeShape<DK, DV>::NW][DK];
    float q[DecodeShape<DK, DV>::NW][DK];
    f4 red[2][DecodeShape<DK, DV>::NW][DecodeShape<DK, DV>::CG][2];
};

// Orders a wave's own LDS writes before its later LDS reads (no other wave
// takes part).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// One token of the rule on the tile slice this thread holds in registers (st):
// normalise q and k (key head rows at qk_off), reduce H^T k^ and H^T q~ over
// dk, write the token's output (row gh of o, v, g, beta) and leave the new tile
// in st. When `out` (a (slot, head) tile) is given, each new row is also
// stored as soon as it is formed, so the stores start while the rest of the
// rows are still being read from LDS. Every wave normalises q and k itself
// into its own LDS copy, so the only workgroup barrier of a token is the one
// exchange of the waves' partial sums; `parity` alternates over a verify
// chain's tokens, so one token's exchange never overwrites what the waves are
// still reading of the previous one. (A wave's LDS operations complete in
// order, so its k^ copy can be rewritten for the next token once read.)
template <int DK, int DV, int DVW, typename T>
__device__ __forceinline__ void token_update(const DecodeParams& p, size_t qk_off, size_t gh, int c0,
                                             f4 (&st)[DecodeShape<DK, DVW>::RPT], TokenScratch<DK, DVW>& sm,
                                             int parity, f4* out) {
    using Sh = DecodeShape<DK, DVW>;
    constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NW = Sh::NW;
    constexpr int KPL = (DK + 63) / 64;   // q/k elements per lane
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid % CG;
    const int rg = tid / CG;

    // L2-normalise k and q in every wave, into the wave's own LDS copy
    float kx[KPL], qx[KPL];
    float sk = 0.f, sq = 0.f, skq = 0.f;
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int i = lane + 64 * e;
        kx[e] = (i < DK) ? Elem<T>::load(p.k, qk_off + i) : 0.f;
        qx[e] = (i < DK) ? Elem<T>::load(p.q, qk_off + i) : 0.f;
        sk += kx[e] * kx[e];
        sq += qx[e] * qx[e];
        skq += kx[e] * qx[e];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        sk += __shfl_xor(sk, off);
        sq += __shfl_xor(sq, off);
        skq += __shfl_xor(skq, off);
    }
    const float rk = 1.0f / sqrtf(sk + p.eps);
    const float rq = p.scale / sqrtf(sq + p.eps);
    const float kq = skq * rk * rq;          // k^ . q~
    const float eg = expf(p.g[gh]);
    const float bt = p.beta[gh];
    const f4 vv = Elem<T>::load4(p.v, gh * DV + c0 + 4 * cg);
    float* kw = sm.k[wave];
    float* qw = sm.q[wave];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int i = lane + 64 * e;
        if (i < DK) {
            kw[i] = kx[e] * rk;
            qw[i] = qx[e] * rq;
        }
    }
    wave_lds_sync();

    // partial H^T k^ and H^T q~ over this thread's rows
    f4 a = f4{0.f, 0.f, 0.f, 0.f};
    f4 c = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + RG * m;
        a += st[m] * kw[row];
        c += st[m] * qw[row];
    }
    // reduce over the row groups: lanes CG apart inside a wave, then the
    // waves through LDS, always in the same order (deterministic)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        a.x += __shfl_xor(a.x, off);
        a.y += __shfl_xor(a.y, off);
        a.z += __shfl_xor(a.z, off);
        a.w += __shfl_xor(a.w, off);
        c.x += __shfl_xor(c.x, off);
        c.y += __shfl_xor(c.y, off);
        c.z += __shfl_xor(c.z, off);
        c.w += __shfl_xor(c.w, off);
    }
    f4 A = a, C = c;
    if constexpr (NW > 1) {
        if (lane < CG) {
            sm.red[parity][wave][lane][0] = a;
            sm.red[parity][wave][lane][1] = c;
        }
        __syncthreads();
        A = sm.red[parity][0][cg][0];
        C = sm.red[parity][0][cg][1];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            A += sm.red[parity][w][cg][0];
            C += sm.red[parity][w][cg][1];
        }
    }

    // delta correction, output, and the new tile
    const f4 u = bt * (vv - eg * A);
    if (rg == 0) Elem<T>::store4(p.o, gh * DV + c0 + 4 * cg, eg * C + kq * u);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + RG * m;
        st[m] = eg * st[m] + kw[row] * u;
        if (out != nullptr) __builtin_nontemporal_store(st[m], out + row * (DV / 4) + c0 / 4 + cg);
    }
}

// load / store of this thread's slice of a (slot, head) tile, 128-bit
// non-temporal (a tile is touched once per launch)
template <int DK, int DV, int DVW>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int slot, int h, int c0,
                                          f4 (&st)[DecodeShape<DK, DVW>::RPT]) {
    using Sh = DecodeShape<DK, DVW>;
    const int cg = threadIdx.x % Sh::CG, rg = threadIdx.x / Sh::CG;
    if (slot >= 0) {
        const f4* in = reinterpret_cast<const f4*>(p.pool + (static_cast<size_t>(slot) * p.hv + h) * (DK * DV) + c0);
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) st[m] = __builtin_nontemporal_load(in + (rg + Sh::RG * m) * (DV / 4) + cg);
    } else {
#pragma unroll
        for (int m = 0; m < Sh::RPT; ++m) st[m] = f4{0.f, 0.f, 0.f, 0.f};
    }
}

// a (slot, head) tile of the pool
__device__ __forceinline__ f4* tile_ptr(const DecodeParams& p, int slot, int h, int elems) {
    return reinterpret_cast<f4*>(p.pool + (static_cast<size_t>(slot) * p.hv + h) * elems);
}

// One workgroup per (request, head, column slice): NS = DV / DVW slices of
// DVW columns. Every column of a tile is its own dk-vector under the rule
// (all of them see the same k^ and q~), so slices are independent; each
// slice's workgroup redoes the small q/k normalisation.
template <int DK, int DV, int DVW, typename T>
__global__ void __launch_bounds__(decode_threads(DK, DVW)) gdn_decode_kernel(DecodeParams p) {
    constexpr int NS = DV / DVW;
    __shared__ TokenScratch<DK, DVW> sm;
    const unsigned tile = blockIdx.x / NS;
    const int c0 = static_cast<int>(blockIdx.x - tile * NS) * DVW;
    const int b = tile / p.hv;
    const int h = tile - b * p.hv;

    const int d = p.dst[b];
    if (d < 0) return;                       // padding row
    const int s = p.src[b];
    if (d >= p.num_slots || s >= p.num_slots) {
        if (threadIdx.x == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    // issue the whole source slice first; the token's small loads overlap its latency
    f4 st[DecodeShape<DK, DVW>::RPT];
    load_tile<DK, DV, DVW>(p, s, h, c0, st);
    const size_t qk_off = (static_cast<size_t>(b) * p.hk + h / p.group) * DK;
    token_update<DK, DV, DVW, T>(p, qk_off, static_cast<size_t>(b) * p.hv + h, c0, st, sm, 0,
                                 tile_ptr(p, d, h, DK * DV));
}

// Speculative-decode verification: draft tokens 0 .. n-1 of request b in
// order on the slice held in registers; the slice goes to dst[b][i] after
// token i when that entry is >= 0. The source is read once for all of them.
// Every token ends in a slice store, so residency hides more latency than
// registers save: the kernel is held to at most 128 VGPRs (four waves per
// SIMD), which measured faster than the uncapped build even where the
// 128-wide slice then spills a few registers.
template <int DK, int DV, int DVW, typename T>
__global__ void __launch_bounds__(decode_threads(DK, DVW)) __attribute__((amdgpu_waves_per_eu(4, 8)))
gdn_verify_kernel(DecodeParams p) {
    constexpr int NS = DV / DVW;
    __shared__ TokenScratch<DK, DVW> sm;
    const unsigned tile = blockIdx.x / NS;
    const int c0 = static_cast<int>(blockIdx.x - tile * NS) * DVW;
    const int b = tile / p.hv;
    const int h = tile - b * p.hv;
    const int K = p.ndraft;
    const int n = p.lens != nullptr ? p.lens[b] : K;
    if (n == 0) return;
    if (n < 0 || n > K) {
        if (threadIdx.x == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_DRAFT_LEN);
        return;
    }
    const int s = p.src[b];
    bool bad = s >= p.num_slots;
    for (int i = 0; i < n; ++i) bad |= p.dst[static_cast<size_t>(b) * K + i] >= p.num_slots;
    if (bad) {
        if (threadIdx.x == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    f4 st[DecodeShape<DK, DVW>::RPT];
    load_tile<DK, DV, DVW>(p, s, h, c0, st);
    const int j = h / p.group;
    for (int i = 0; i < n; ++i) {
        const size_t t = static_cast<size_t>(b) * K + i;      // token row
        const int d = p.dst[t];
        token_update<DK, DV, DVW, T>(p, (t * p.hk + j) * DK, t * p.hv + h, c0, st, sm, i & 1,
                                     d >= 0 ? tile_ptr(p, d, h, DK * DV) : nullptr);
    }
}

template <int DK, int DV, int DVW, typename T, bool VERIFY>
int launch_shape(const DecodeParams& p, int batch, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(batch) * static_cast<unsigned>(p.hv) * static_cast<unsigned>(DV / DVW));
    const dim3 block(DecodeShape<DK, DVW>::NT);
    if (VERIFY) hipLaunchKernelGGL((gdn_verify_kernel<DK, DV, DVW, T>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gdn_decode_kernel<DK, DV, DVW, T>), grid, block, 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string(VERIFY ? "gdn_decode_verify" : "gdn_decode_step") + ": launch failed: " +
                                        hipGetErrorString(e));
    return GDN_OK;
}

// Column slices per tile. A launch has batch * HV tiles and MI355X has 256
// CUs; a small batch leaves most of them idle while each workgroup streams a
// whole 64 KiB tile. Measured on MI355X at HV = 32, 128 x 128 (in-place bf16
// decode): 4 slices are fastest up to 64 tiles (B = 1: 3.7 us against 4.6 us
// whole), 2 slices below 512 tiles (B = 8: 5.8 against 6.9 us), whole tiles
// from 512 up (B = 16: 9.7 against 11.5 us split in 2). A slice keeps at
// least 32 columns so each of its rows is a whole 128-byte line: 16-column
// slices, which share lines between workgroups, were slower at every batch.
int decode_split(int64_t tiles, int dv) {
    int s = 1;
    if (tiles < 512) s = 2;
    if (tiles <= 64) s = 4;
    while (s > 1 && dv / s < 32) s /= 2;
    return s;
}

template <int DK, int DV, typename T, bool VERIFY>
int launch_split(const DecodeParams& p, int batch, int split, hipStream_t s) {
    if constexpr (DV / 4 >= 32)
        if (split == 4) return launch_shape<DK, DV, DV / 4, T, VERIFY>(p, batch, s);
    if constexpr (DV / 2 >= 32)
        if (split == 2) return launch_shape<DK, DV, DV / 2, T, VERIFY>(p, batch, s);
    return launch_shape<DK, DV, DV, T, VERIFY>(p, batch, s);
}

template <typename T, bool VERIFY>
int dispatch_dv(const DecodeParams& p, int batch, int dk, int dv, hipStream_t s) {
    const int split = decode_split(static_cast<int64_t>(batch) * p.hv, dv);
#define GDN_DK_CASE(DK)                                                             \
    if (dk == DK) {                                                                 \
        switch (dv) {                                                               \
            case 16: return launch_split<DK, 16, T, VERIFY>(p, batch, split, s);    \
            case 32: return launch_split<DK, 32, T, VERIFY>(p, batch, split, s);    \
            case 64: return launch_split<DK, 64, T, VERIFY>(p, batch, split, s);    \
            case 128: return launch_split<DK, 128, T, VERIFY>(p, batch, split, s);  \
            default: break;                                                         \
        }                                                                           \
    }
    GDN_DK_CASE(16)
    GDN_DK_CASE(32)
    GDN_DK_CASE(64)
    GDN_DK_CASE(128)
#undef GDN_DK_CASE
    return gdn::fail(GDN_E_UNSUPPORTED, std::string(VERIFY ? "gdn_decode_verify" : "gdn_decode_step") + ": unsupported dk/dv");
}

template <typename A>
DecodeParams make_params(const gdn_pool* pool, const A* a) {
    DecodeParams p;
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.g = a->g;
    p.beta = a->beta;
    p.o = a->o;
    p.pool = pool->storage;
    p.src = a->src_slots;
    p.dst = a->dst_slots;
    p.err = a->err_flag;
    p.hk = a->num_k_heads;
    p.hv = a->num_v_heads;
    p.group = a->num_v_heads / a->num_k_heads;
    p.num_slots = pool->num_slots;
    p.scale = a->scale;
    p.eps = a->l2_eps;
    p.ndraft = 1;
    p.lens = nullptr;
    return p;
}

}  // namespace

namespace gdn {

int launch_decode(const gdn_pool* pool, const gdn_decode_args* a, void* stream, float* storage) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    DecodeParams p = make_params(pool, a);
    if (storage != nullptr) p.pool = storage;
    if (a->dtype == GDN_DTYPE_F32) return dispatch_dv<float, false>(p, a->batch, a->dk, a->dv, s);
    return dispatch_dv<uint16_t, false>(p, a->batch, a->dk, a->dv, s);
}

int launch_verify(const gdn_pool* pool, const gdn_verify_args* a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    DecodeParams p = make_params(pool, a);
    p.ndraft = a->num_draft;
    p.lens = a->draft_lens;
    if (a->dtype == GDN_DTYPE_F32) return dispatch_dv<float, true>(p, a->batch, a->dk, a->dv, s);
    return dispatch_dv<uint16_t, true>(p, a->batch, a->dk, a->dv, s);
}

}  // namespace gdn
