// Prefill of float32 inputs: the gated delta rule token by token in fp32.
//
// The chunked form of the bf16 prefill feeds its products to bf16 matrix
// cores; with float32 inputs that rounding would dominate the error, so
// float32 sequences run the per-token rule directly (the same arithmetic as
// decode), with the state held in registers for the whole sequence:
//
//   a = H^T k^,  c = H^T q~,  u = beta (v - exp(g) a),
//   o = exp(g) c + u (k^ . q~),  H' = exp(g) H + k^ u^T.
//
// One wavefront per (sequence, value head, column slice of 4, 8 or 16
// columns): the columns of H are independent under the rule, so the slices
// are too, and thin slices let a single long sequence occupy the chip. Each
// lane holds a few consecutive rows of its slice and loads those rows of k
// and q itself, so the per-token work needs no LDS and no barrier: the sums
// over dk are DPP and lane-swap reductions inside the wavefront. The next
// token's inputs are loaded while the current one runs. The slice goes to
// the checkpoint slots at the chosen 64-token chunk ends and to the
// destination at the end; source slots are only read (copy-on-write, as in
// the TokenSpeed article, 24-ai.news, English, section "What are the key
// optimizations behind the record?").

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gdn_internal.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

struct TokenParams {
    const float* q;
    const float* k;
    const float* v;
    const float* g;
    const float* beta;
    float* o;
    float* pool;
    const int32_t* cu;
    const int32_t* src;
    const int32_t* dst;
    const int32_t* ckpt;        // optional [chunks] checkpoint slots
    const int32_t* chunk_off;   // [N + 1] first chunk of each sequence (when ckpt)
    int32_t* chunk_off_w;
    int32_t* err;
    int32_t hk, hv, group, num_slots, n_seqs;
    float scale, eps;
};

// First 64-token chunk of every sequence (exclusive prefix sum of
// ceil(len / 64)), 1024 sequences per round: a scan inside each wave, then
// the wave totals through LDS.
constexpr int kOffThreads = 1024;

__global__ void __launch_bounds__(kOffThreads) token_chunk_offsets_kernel(TokenParams p) {
    constexpr int NWV = kOffThreads / 64;
    __shared__ int wsum[NWV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int carry = 0;
    for (int base = 0; base < p.n_seqs; base += kOffThreads) {
        const int i = base + tid;
        int nc = 0;
        if (i < p.n_seqs) nc = (p.cu[i + 1] - p.cu[i] + 63) / 64;
        int x = nc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        int o = carry, t = 0;
#pragma unroll
        for (int k = 0; k < NWV; ++k) {
            if (k < w) o += wsum[k];
            t += wsum[k];
        }
        if (i < p.n_seqs) p.chunk_off_w[i] = o + x - nc;
        carry += t;
        __syncthreads();                        // wsum is rewritten next round
    }
    if (tid == 0) p.chunk_off_w[p.n_seqs] = carry;
}

// Tokens of inputs in flight: 4 for the thinnest slices (one wavefront per
// SIMD, registers to spare; 7 % faster on one 8192-token sequence than 2),
// 2 for wider ones, which run two wavefronts per SIMD and would lose one of
// them to the extra registers.
constexpr int tokens_ahead(int cols) { return cols <= 4 ? 4 : 2; }

// Lane layout of a COLS-column slice of a dk x dv tile: CG float4 column
// groups and RG = 64 / CG row groups; lane l = rg * CG + cg holds column
// group cg of the RPT consecutive rows rg * RPT .. rg * RPT + RPT - 1, and
// loads those rows of k and q itself. The lanes sharing cg (a "class") hold
// every row once, so sums over a class are sums over dk.
template <int DK, int COLS>
struct Slice {
    static constexpr int CG = COLS / 4;
    static constexpr int RG = 64 / CG;
    static constexpr int RPT = DK / RG;   // rows per lane
    static_assert(COLS % 4 == 0 && 64 % CG == 0 && DK % RG == 0 && RPT >= 1, "unsupported slice");
};

template <int RPT>
struct TokenIn {
    float k[RPT], q[RPT];   // this lane's rows of k and q
    f4 v;                   // this lane's column group of v
    float g, beta;
};

template <int N>
__device__ __forceinline__ void load_rows(const float* p, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f4 w = *reinterpret_cast<const f4*>(p + i);
            x[i] = w.x;
            x[i + 1] = w.y;
            x[i + 2] = w.z;
            x[i + 3] = w.w;
        }
    } else if constexpr (N == 2) {
        const float2 w = *reinterpret_cast<const float2*>(p);
        x[0] = w.x;
        x[1] = w.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = p[i];
    }
}

template <int DK, int DV, int COLS>
__device__ __forceinline__ void fetch_token(const TokenParams& p, int t, int j, int h, int c0, int lane,
                                            TokenIn<Slice<DK, COLS>::RPT>& in) {
    using S = Slice<DK, COLS>;
    const int rg = lane / S::CG, cg = lane % S::CG;
    const size_t r = (static_cast<size_t>(t) * p.hk + j) * DK + rg * S::RPT;
    load_rows(p.k + r, in.k);
    load_rows(p.q + r, in.q);
    const size_t gh = static_cast<size_t>(t) * p.hv + h;
    in.v = *reinterpret_cast<const f4*>(p.v + gh * DV + c0 + 4 * cg);
    in.g = p.g[gh];
    in.beta = p.beta[gh];
}

// Cross-lane sums without LDS: DPP inside 16-lane rows, then the gfx950 row
// and half swaps. A swap exchanges data between lane groups of its two
// operands; with both operands equal, the sum of its two results is the sum
// over the group pair, whichever half lands where.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum_row_pairs(float x) {    // lanes 16 apart
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sum_halves(float x) {       // lanes 32 apart
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kRowRor4 = 0x124;   // rotate right by 4 inside a row
constexpr int kRowRor8 = 0x128;   // rotate right by 8 inside a row

// sum over the lanes that share lane % CG (CG in 1, 2, 4): every lane ends
// with the sum of its class
template <int CG>
__device__ __forceinline__ float sum_classes(float x) {
    if constexpr (CG == 1) x += dpp<kQuadXor1>(x);
    if constexpr (CG <= 2) x += dpp<kQuadXor2>(x);
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor8>(x);
    return sum_halves(sum_row_pairs(x));
}

template <int DK, int DV, int COLS>
__device__ __forceinline__ void store_slice(const TokenParams& p, int slot, int h, int c0, int lane,
                                            const f4 (&st)[Slice<DK, COLS>::RPT]) {
    using S = Slice<DK, COLS>;
    f4* out = reinterpret_cast<f4*>(p.pool + (static_cast<size_t>(slot) * p.hv + h) * (DK * DV) + c0);
    const int cg = lane % S::CG, rg = lane / S::CG;
#pragma unroll
    for (int m = 0; m < S::RPT; ++m) out[(rg * S::RPT + m) * (DV / 4) + cg] = st[m];
}

template <int DK, int DV, int COLS>
__global__ void __launch_bounds__(64) prefill_tokens_kernel(TokenParams p) {
    using S = Slice<DK, COLS>;
    static_assert(DV % COLS == 0, "unsupported tile shape");
    constexpr int NS = DV / COLS;
    constexpr int kAhead = tokens_ahead(COLS);
    constexpr int CG = S::CG, RPT = S::RPT;
    const int lane = threadIdx.x & 63;                // one wavefront per workgroup
    const unsigned tile = blockIdx.x / NS;
    const int c0 = static_cast<int>(blockIdx.x - tile * NS) * COLS;
    const int n = tile / p.hv;
    const int h = tile - n * p.hv;
    const int cg = lane % CG, rg = lane / CG;

    const int d = p.dst[n];
    if (d < 0) return;                                // sequence skipped
    const int s = p.src[n];
    if (d >= p.num_slots || s >= p.num_slots) {
        if (lane == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    f4 st[RPT];
    if (s >= 0) {
        const f4* in = reinterpret_cast<const f4*>(p.pool + (static_cast<size_t>(s) * p.hv + h) * (DK * DV) + c0);
#pragma unroll
        for (int m = 0; m < RPT; ++m) st[m] = in[(rg * RPT + m) * (DV / 4) + cg];
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) st[m] = f4{0.f, 0.f, 0.f, 0.f};
    }

    const int t0 = p.cu[n], t1 = p.cu[n + 1];
    const int j = h / p.group;
    const int cbase = p.ckpt != nullptr ? p.chunk_off[n] : 0;

    // Output row of the previous token, stored only after this token's inputs
    // have arrived: a store issued between a load and its first use would be
    // waited for along with the load (memory operations retire in order).
    f4 o_prev = f4{0.f, 0.f, 0.f, 0.f};
    auto store_o = [&](int t) {
        if (rg == 0) *reinterpret_cast<f4*>(p.o + (static_cast<size_t>(t) * p.hv + h) * DV + c0 + 4 * cg) = o_prev;
    };

    // One token; `nxt` (the buffer token t - 1 used) receives the inputs of
    // token t + kAhead - 1 while this one runs. Past the end the last token
    // is loaded again: an unconditional load keeps the wait counts exact.
    // H^T k and H^T q are formed on the raw k and q, beside the norms, and
    // scaled afterwards, so the state chain does not wait for the norms.
    auto step = [&](int t, const TokenIn<RPT>& cur, TokenIn<RPT>& nxt) {
        const int tn = t + kAhead - 1;
        fetch_token<DK, DV, COLS>(p, tn < t1 ? tn : t1 - 1, j, h, c0, lane, nxt);

        float s_kk = 0.f, s_qq = 0.f, s_kq = 0.f;
        f4 a = f4{0.f, 0.f, 0.f, 0.f};
        f4 c = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            s_kk += cur.k[m] * cur.k[m];
            s_qq += cur.q[m] * cur.q[m];
            s_kq += cur.k[m] * cur.q[m];
            a += st[m] * cur.k[m];
            c += st[m] * cur.q[m];
        }
        s_kk = sum_classes<CG>(s_kk);
        s_qq = sum_classes<CG>(s_qq);
        s_kq = sum_classes<CG>(s_kq);
        a.x = sum_classes<CG>(a.x);
        a.y = sum_classes<CG>(a.y);
        a.z = sum_classes<CG>(a.z);
        a.w = sum_classes<CG>(a.w);
        c.x = sum_classes<CG>(c.x);
        c.y = sum_classes<CG>(c.y);
        c.z = sum_classes<CG>(c.z);
        c.w = sum_classes<CG>(c.w);
        // hardware reciprocal square root and base-2 exponential (about
        // 1 ulp each, far inside the fp32 accuracy bar of this path)
        const float rk = __builtin_amdgcn_rsqf(s_kk + p.eps);
        const float rq = p.scale * __builtin_amdgcn_rsqf(s_qq + p.eps);
        const float kq = s_kq * rk * rq;
        const float eg = __builtin_amdgcn_exp2f(cur.g * 1.44269504088896341f);
        if (t > t0) store_o(t - 1);

        // u = beta (v - e^g H^T k^), o = e^g H^T q~ + (k^ . q~) u, H <- e^g H + k^ u^T
        const f4 u = cur.beta * (cur.v - (eg * rk) * a);
        o_prev = (eg * rq) * c + kq * u;
#pragma unroll
        for (int m = 0; m < RPT; ++m) st[m] = eg * st[m] + (cur.k[m] * rk) * u;

        if (p.ckpt != nullptr) {
            const int r = t - t0 + 1;                  // tokens done in this sequence
            if ((r & 63) == 0 || t + 1 == t1) {
                const int slot = p.ckpt[cbase + (r - 1) / 64];
                if (slot >= p.num_slots) {
                    if (lane == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
                } else if (slot >= 0) {
                    store_slice<DK, DV, COLS>(p, slot, h, c0, lane, st);
                }
            }
        }
    };

    // A ring of kAhead input buffers, indexed at compile time (no register
    // copies between tokens).
    if (t1 > t0) {
        TokenIn<RPT> ring[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead - 1; ++i)
            fetch_token<DK, DV, COLS>(p, t0 + i < t1 ? t0 + i : t1 - 1, j, h, c0, lane, ring[i]);
        int t = t0;
        for (; t + kAhead <= t1; t += kAhead) {
#pragma unroll
            for (int i = 0; i < kAhead; ++i) step(t + i, ring[i], ring[(i + kAhead - 1) % kAhead]);
        }
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
            if (t + i < t1) step(t + i, ring[i], ring[(i + kAhead - 1) % kAhead]);
        store_o(t1 - 1);
    }
    store_slice<DK, DV, COLS>(p, d, h, c0, lane, st);
}

int check(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked: ") + what + " launch failed: " +
                                        hipGetErrorString(e));
    return GDN_OK;
}

template <int DK, int DV, int COLS>
int launch_cols(const TokenParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.n_seqs) * static_cast<unsigned>(p.hv) * (DV / COLS));
    hipLaunchKernelGGL((prefill_tokens_kernel<DK, DV, COLS>), grid, dim3(64), 0, s, p);
    return check("fp32 token recurrence");
}

// Slice width. A wavefront's time per token is set by the instructions it
// issues, which scale with the rows x columns it holds, so a call with few
// (sequence, head) pairs cuts the heads into thinner slices: 16 columns
// while that gives 2048 wavefronts (2 per SIMD), else 8, else 4. A slice
// needs at least one row per lane group: dk * cols >= 256.
constexpr int64_t kWaveTarget = 2048;

template <int DK, int DV>
int launch_tokens(const TokenParams& p, hipStream_t s) {
    const int64_t pairs = static_cast<int64_t>(p.n_seqs) * p.hv;
    if constexpr (DV >= 16 && DK * 16 >= 256)
        if (pairs * (DV / 16) >= kWaveTarget || DK * 8 < 256) return launch_cols<DK, DV, 16>(p, s);
    if constexpr (DK * 8 >= 256)
        if (pairs * (DV / 8) >= kWaveTarget || DK * 4 < 256) return launch_cols<DK, DV, 8>(p, s);
    if constexpr (DK * 4 >= 256) return launch_cols<DK, DV, 4>(p, s);
    return launch_cols<DK, DV, 16>(p, s);
}

template <int DK>
int launch_dv(const TokenParams& p, int dv, hipStream_t s) {
    switch (dv) {
        case 16: return launch_tokens<DK, 16>(p, s);
        case 32: return launch_tokens<DK, 32>(p, s);
        case 64: return launch_tokens<DK, 64>(p, s);
        case 128: return launch_tokens<DK, 128>(p, s);
        default: return gdn::fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dv");
    }
}

}  // namespace

namespace gdn {

int launch_prefill_f32(const gdn_pool* pool, const gdn_prefill_args* a, const PrefillPlan& plan, void* workspace,
                       void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    TokenParams p;
    p.q = static_cast<const float*>(a->q);
    p.k = static_cast<const float*>(a->k);
    p.v = static_cast<const float*>(a->v);
    p.g = a->g;
    p.beta = a->beta;
    p.o = static_cast<float*>(a->o);
    p.pool = pool->storage;
    p.cu = a->cu_seqlens;
    p.src = a->src_slots;
    p.dst = a->dst_slots;
    p.ckpt = a->ckpt_slots;
    p.chunk_off = reinterpret_cast<const int32_t*>(ws + plan.off_chunk_offsets);
    p.chunk_off_w = reinterpret_cast<int32_t*>(ws + plan.off_chunk_offsets);
    p.err = a->err_flag;
    p.hk = a->num_k_heads;
    p.hv = a->num_v_heads;
    p.group = a->num_v_heads / a->num_k_heads;
    p.num_slots = pool->num_slots;
    p.n_seqs = a->num_seqs;
    p.scale = a->scale;
    p.eps = a->l2_eps;
    if (p.ckpt != nullptr) {
        hipLaunchKernelGGL(token_chunk_offsets_kernel, dim3(1), dim3(kOffThreads), 0, s, p);
        const int st = check("chunk-offset");
        if (st != GDN_OK) return st;
    }
    switch (a->dk) {
        case 16: return launch_dv<16>(p, a->dv, s);
        case 32: return launch_dv<32>(p, a->dv, s);
        case 64: return launch_dv<64>(p, a->dv, s);
        case 128: return launch_dv<128>(p, a->dv, s);
        default: return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dk");
    }
}

}  // namespace gdn
