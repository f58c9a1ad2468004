// Chunked prefill of the gated delta rule over a slot pool (gfx950).
//
// Every sequence (packed by cu_seqlens) is cut into chunks of C = 64 tokens,
// restarting at each sequence boundary. Inside a chunk of c tokens, with
// cumulative log-decay gamma_r = sum_{s<=r} g_s, k^/q~ the normalised keys and
// scaled queries, and H the dk x dv state at the chunk start (H = S^T), the
// token recurrence is exactly
//
//   A[r,s] = beta_r exp(gamma_r - gamma_s) (k^_r . k^_s)   (s < r)
//   T      = (I + A)^-1                                    (unit lower triangular)
//   U      = T diag(beta) (V - diag(exp(gamma)) K^ H)      (the per-token updates u_r)
//   P[r,s] = exp(gamma_r - gamma_s) (q~_r . k^_s)          (s <= r)
//   O      = diag(exp(gamma)) Q~ H + P U
//   H'     = exp(gamma_last) H + K^T diag(exp(gamma_last - gamma)) U
//
// (the WY / UT form: U = U' - W H with W = T diag(beta exp(gamma)) K^ and
// U' = T diag(beta) V, here applied as T times one bracket). Decay factors are
// always exp of a non-positive difference.
//
// Two kernels after a tiny chunk-offset prep:
//  * intra-chunk, one wave per (chunk, value head), fully parallel: row norms,
//    the Gram matrices K K^T and Q K^T on bf16 MFMA (exact bf16 products, fp32
//    accumulation), A staged in LDS, T by forward substitution in fp32 with
//    the column in registers, and P, T, per-token scale factors and a
//    transposed copy of the raw K tile written to the workspace;
//  * recurrence, one workgroup per (sequence, value head, 16*NW value
//    columns), sequential over the chunks of its sequence: each wave keeps
//    its 16 columns of the fp32 master state in MFMA accumulators and runs
//    X = K H, Z = Q H, U = T Y, O = scale Z + P U and H' = e H + K^T (D U) as
//    bf16 MFMA contractions (16x16x32), with the chunk's operands staged
//    through LDS. MFMA operands are bf16; accumulators and the state are fp32.
//
// Raw (unnormalised) bf16 q and k are the MFMA operands; the L2 norms and the
// decay factors are applied as fp32 row scales on the accumulator side.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gdn_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kC = 64;        // chunk length
constexpr int kScStride = 5;  // per-token scale rows in the workspace

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
    uint16_t* kt;               // [chunks][HK][DK][64]   raw K^T per chunk
    uint16_t* tp;               // [chunks][HV][2][64][64] T then P
    float* sc;                  // [chunks][HV][5][64]    scale factors
    int32_t* chunk_off_w;       // same buffer as chunk_off, written by the prep kernel
    int32_t n_seqs;
    int32_t num_chunks;
    int32_t total_tokens;
    int32_t hk;
    int32_t hv;
    int32_t group;
    int32_t dv;
    int32_t num_slots;
    float scale;
    float eps;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// 8 bf16 from two fp32 accumulator quads: slots 0-3 <- a, 4-7 <- b.
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
    u32x4 w;
    w.x = pack_bf16x2(a.x, a.y);
    w.y = pack_bf16x2(a.z, a.w);
    w.z = pack_bf16x2(b.x, b.y);
    w.w = pack_bf16x2(b.z, b.w);
    return as_bf16x8(w);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MFMA operand read from a row-major bf16 LDS tile with the K-slot order that
// matches an accumulator pair: slots 0-3 hold columns base+4g..+3 and slots
// 4-7 columns base+16+4g..+3 (g = lane / 16). An fp32 accumulator tile pair
// (rows base..base+15, base+16..base+31) packed with pack8 has exactly this
// order, so either side can feed the other without a shuffle.
__device__ __forceinline__ bf16x8 lds_pair(const uint16_t* buf, int stride, int row, int base, int g4) {
    const uint16_t* p = buf + row * stride + base + 4 * g4;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
    u32x4 w;
    w.x = lo.x;
    w.y = lo.y;
    w.z = hi.x;
    w.w = hi.y;
    return as_bf16x8(w);
}

// 8 consecutive bf16 (contiguous K-slot order).
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* buf, int stride, int row, int base) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + row * stride + base));
}

// ---------------------------------------------------------------------------
// prep: first chunk index of every sequence
// ---------------------------------------------------------------------------

__global__ void chunk_offsets_kernel(PrefillParams p) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int32_t acc = 0;
    for (int i = 0; i < p.n_seqs; ++i) {
        p.chunk_off_w[i] = acc;
        const int32_t len = p.cu[i + 1] - p.cu[i];
        acc += len > 0 ? (len + kC - 1) / kC : 0;
    }
    p.chunk_off_w[p.n_seqs] = acc;
}

// Locate chunk c: the last sequence n with chunk_off[n] <= c.
__device__ __forceinline__ int find_seq(const int32_t* off, int n_seqs, int c) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// intra-chunk: one wave per (chunk, value head)
// ---------------------------------------------------------------------------

template <int DK>
__global__ void __launch_bounds__(64) prefill_intra_kernel(PrefillParams p) {
    constexpr int KS = DK / 32;       // MFMA k-steps over dk
    constexpr int SK = DK + 8;        // LDS row stride of the q/k tiles (bf16)
    constexpr int SA = kC + 4;        // LDS row stride of A (fp32)
    __shared__ __align__(16) uint16_t sK[kC * SK];
    __shared__ __align__(16) uint16_t sQ[kC * SK];
    __shared__ __align__(16) float sA[kC * SA];
    __shared__ float sGam[kC], sBeta[kC], sRk[kC], sRq[kC];

    const int c = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int g4 = lane >> 4, l16 = lane & 15;
    if (c >= p.num_chunks) return;
    const int n = find_seq(p.chunk_off, p.n_seqs, c);
    const int t0 = p.cu[n] + (c - p.chunk_off[n]) * kC;
    const int tend = p.cu[n + 1];
    const int len = min(kC, tend - t0);
    if (len <= 0 || tend > p.total_tokens || p.dst[n] < 0) return;
    const int j = h / p.group;

    // stage the raw q / k rows of the chunk (zero rows past the end)
    for (int idx = lane; idx < kC * (DK / 8); idx += 64) {
        const int r = idx / (DK / 8), c8 = idx % (DK / 8);
        u32x4 kv = u32x4{0u, 0u, 0u, 0u}, qv = u32x4{0u, 0u, 0u, 0u};
        if (r < len) {
            const size_t off = (static_cast<size_t>(t0 + r) * p.hk + j) * DK + c8 * 8;
            kv = *reinterpret_cast<const u32x4*>(p.k + off);
            qv = *reinterpret_cast<const u32x4*>(p.q + off);
        }
        *reinterpret_cast<u32x4*>(sK + r * SK + c8 * 8) = kv;
        *reinterpret_cast<u32x4*>(sQ + r * SK + c8 * 8) = qv;
    }
    // per-token g, beta; cumulative log-decay by an inclusive lane scan
    float gl = 0.f, bl = 0.f;
    if (lane < len) {
        const size_t gi = static_cast<size_t>(t0 + lane) * p.hv + h;
        gl = p.g[gi];
        bl = p.beta[gi];
    }
    float gam = gl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(gam, off);
        if (lane >= off) gam += t;
    }
    const float gam_last = __shfl(gam, 63);   // padded tokens add g = 0
    __syncthreads();

    // L2 norms of row `lane` (fp32 sums of exact bf16 squares)
    float sk = 0.f, sq = 0.f;
    for (int d8 = 0; d8 < DK / 8; ++d8) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(sK + lane * SK + d8 * 8);
        const u32x4 qv = *reinterpret_cast<const u32x4*>(sQ + lane * SK + d8 * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float k0 = __uint_as_float(kv[e] << 16), k1 = __uint_as_float(kv[e] & 0xffff0000u);
            const float q0 = __uint_as_float(qv[e] << 16), q1 = __uint_as_float(qv[e] & 0xffff0000u);
            sk += k0 * k0 + k1 * k1;
            sq += q0 * q0 + q1 * q1;
        }
    }
    const bool live = lane < len;
    const float rk = live ? 1.0f / sqrtf(sk + p.eps) : 0.f;
    const float rq = live ? p.scale / sqrtf(sq + p.eps) : 0.f;
    sGam[lane] = gam;
    sBeta[lane] = bl;
    sRk[lane] = rk;
    sRq[lane] = rq;
    {
        float* scp = p.sc + (static_cast<size_t>(c) * p.hv + h) * (kScStride * kC);
        const float eg = expf(gam);
        scp[0 * kC + lane] = eg * rk;                      // row scale of K H
        scp[1 * kC + lane] = bl;                           // beta
        scp[2 * kC + lane] = eg * rq;                      // row scale of Q H
        scp[3 * kC + lane] = rk * expf(gam_last - gam);    // row scale of U in the state advance
        scp[4 * kC + lane] = expf(gam_last);               // state decay over the chunk
    }
    __syncthreads();

    // Gram matrices on MFMA, lower-triangular 16x16 tiles; A -> LDS, P -> global
    uint16_t* Pg = p.tp + ((static_cast<size_t>(c) * p.hv + h) * 2 + 1) * (kC * kC);
    for (int tr = 0; tr < 4; ++tr) {
        for (int ts = 0; ts < 4; ++ts) {
            if (ts > tr) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Pg[(16 * tr + 4 * g4 + i) * kC + 16 * ts + l16] = 0;
                continue;
            }
            f32x4 kk = f32x4{0.f, 0.f, 0.f, 0.f}, qk = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = lds_row8(sK, SK, 16 * tr + l16, 32 * ks + 8 * g4);
                const bf16x8 aq = lds_row8(sQ, SK, 16 * tr + l16, 32 * ks + 8 * g4);
                const bf16x8 bk = lds_row8(sK, SK, 16 * ts + l16, 32 * ks + 8 * g4);
                kk = mfma16(ak, bk, kk);
                qk = mfma16(aq, bk, qk);
            }
            const int s = 16 * ts + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tr + 4 * g4 + i;
                const float dec = (s <= r) ? expf(sGam[r] - sGam[s]) : 0.f;
                sA[r * SA + s] = (s < r) ? sBeta[r] * dec * kk[i] * sRk[r] * sRk[s] : 0.f;
                Pg[r * kC + s] = f32_to_bf16(dec * qk[i] * sRq[r] * sRk[s]);
            }
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution; lane t owns column t (rows
    // above t come out zero). A row r is read as float4s; its entries at
    // s >= r are zero inside the diagonal tile, and tc[s >= r] is still zero.
    // The address of row r is made to depend on tc[r - 2] through an empty
    // asm, so at most two rows of A are in registers at a time (otherwise the
    // scheduler hoists all 2016 loads and spills).
    float tc[kC];
#pragma unroll
    for (int r = 0; r < kC; ++r) tc[r] = 0.f;
#pragma unroll
    for (int r = 0; r < kC; ++r) {
        int row_off = r * SA;
        if (r >= 2) __asm__ volatile("" : "+v"(row_off) : "v"(tc[r - 2]));
        const float* arow = sA + row_off;
        float acc = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < (r + 3) / 4; ++q4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(arow + 4 * q4);
            acc += a.x * tc[4 * q4] + a.y * tc[4 * q4 + 1] + a.z * tc[4 * q4 + 2] + a.w * tc[4 * q4 + 3];
        }
        tc[r] = (r == lane) ? 1.f : -acc;
    }
    uint16_t* Tg = p.tp + (static_cast<size_t>(c) * p.hv + h) * 2 * (kC * kC);
#pragma unroll
    for (int r = 0; r < kC; ++r) Tg[r * kC + lane] = f32_to_bf16(tc[r]);

    // raw K^T of the chunk, once per key head
    if (h % p.group == 0) {
        uint16_t* Ktg = p.kt + (static_cast<size_t>(c) * p.hk + j) * (DK * kC);
        for (int d = 0; d < DK; ++d) Ktg[d * kC + lane] = sK[lane * SK + d];
    }
}

// ---------------------------------------------------------------------------
// recurrence: one workgroup per (sequence, value head, 16*NW value columns)
// ---------------------------------------------------------------------------

template <int DK, int NW>
__global__ void __launch_bounds__(64 * NW) prefill_recurrent_kernel(PrefillParams p) {
    constexpr int KS = DK / 32;       // k-steps over dk
    constexpr int MT = DK / 16;       // 16-row tiles of the state
    constexpr int SK = DK + 8;        // q/k tile row stride (bf16)
    constexpr int ST = kC + 8;        // K^T, T, P row stride (bf16)
    constexpr int NV = 16 * NW;       // value columns per workgroup
    constexpr int SV = NV + 8;        // v tile row stride (bf16)
    constexpr int NT = 64 * NW;
    __shared__ __align__(16) uint16_t sK[kC * SK];
    __shared__ __align__(16) uint16_t sQ[kC * SK];
    __shared__ __align__(16) uint16_t sKt[DK * ST];
    __shared__ __align__(16) uint16_t sT[kC * ST];
    __shared__ __align__(16) uint16_t sP[kC * ST];
    __shared__ __align__(16) uint16_t sV[kC * SV];
    __shared__ __align__(16) float sSc[kScStride * kC];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int groups = p.dv / NV;
    const int h = blockIdx.x / groups;
    const int grp = blockIdx.x - h * groups;
    const int n = blockIdx.y;
    const int j = h / p.group;

    const int dsl = p.dst[n];
    if (dsl < 0) return;
    const int ssl = p.src[n];
    const int tb = p.cu[n], te = p.cu[n + 1];
    const int c0 = p.chunk_off[n], c1 = p.chunk_off[n + 1];
    if (dsl >= p.num_slots || ssl >= p.num_slots || te > p.total_tokens || te < tb || c1 > p.num_chunks) {
        if (tid == 0 && p.err != nullptr) atomicOr(p.err, GDN_ERRFLAG_SLOT_RANGE);
        return;
    }
    const int vcol0 = grp * NV;                 // first value column of the workgroup
    const int col = vcol0 + wave * 16 + l16;    // this lane's value column

    // fp32 master state: H[mu][i] = H[16 mu + 4 g + i][col]
    f32x4 H[MT];
    if (ssl >= 0) {
        const float* st = p.pool + (static_cast<size_t>(ssl) * p.hv + h) * (static_cast<size_t>(DK) * p.dv);
#pragma unroll
        for (int mu = 0; mu < MT; ++mu)
#pragma unroll
            for (int i = 0; i < 4; ++i) H[mu][i] = st[(16 * mu + 4 * g4 + i) * p.dv + col];
    } else {
#pragma unroll
        for (int mu = 0; mu < MT; ++mu) H[mu] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int c = c0; c < c1; ++c) {
        const int t0 = tb + (c - c0) * kC;
        const int len = min(kC, te - t0);
        __syncthreads();   // every wave is done with the previous chunk's tiles
        for (int idx = tid; idx < kC * (DK / 8); idx += NT) {
            const int r = idx / (DK / 8), c8 = idx % (DK / 8);
            u32x4 kv = u32x4{0u, 0u, 0u, 0u}, qv = u32x4{0u, 0u, 0u, 0u};
            if (r < len) {
                const size_t off = (static_cast<size_t>(t0 + r) * p.hk + j) * DK + c8 * 8;
                kv = *reinterpret_cast<const u32x4*>(p.k + off);
                qv = *reinterpret_cast<const u32x4*>(p.q + off);
            }
            *reinterpret_cast<u32x4*>(sK + r * SK + c8 * 8) = kv;
            *reinterpret_cast<u32x4*>(sQ + r * SK + c8 * 8) = qv;
        }
        const uint16_t* Ktg = p.kt + (static_cast<size_t>(c) * p.hk + j) * (DK * kC);
        for (int idx = tid; idx < DK * (kC / 8); idx += NT) {
            const int d = idx / (kC / 8), c8 = idx % (kC / 8);
            *reinterpret_cast<u32x4*>(sKt + d * ST + c8 * 8) = *reinterpret_cast<const u32x4*>(Ktg + d * kC + c8 * 8);
        }
        const uint16_t* TPg = p.tp + (static_cast<size_t>(c) * p.hv + h) * 2 * (kC * kC);
        for (int idx = tid; idx < 2 * kC * (kC / 8); idx += NT) {
            const int which = idx / (kC * kC / 8);
            const int rem = idx - which * (kC * kC / 8);
            const int r = rem / (kC / 8), c8 = rem % (kC / 8);
            uint16_t* dstp = (which ? sP : sT) + r * ST + c8 * 8;
            *reinterpret_cast<u32x4*>(dstp) = *reinterpret_cast<const u32x4*>(TPg + which * (kC * kC) + r * kC + c8 * 8);
        }
        for (int idx = tid; idx < kC * (NV / 8); idx += NT) {
            const int r = idx / (NV / 8), c8 = idx % (NV / 8);
            u32x4 vv = u32x4{0u, 0u, 0u, 0u};
            if (r < len)
                vv = *reinterpret_cast<const u32x4*>(p.v + (static_cast<size_t>(t0 + r) * p.hv + h) * p.dv + vcol0 + c8 * 8);
            *reinterpret_cast<u32x4*>(sV + r * SV + c8 * 8) = vv;
        }
        const float* SCg = p.sc + (static_cast<size_t>(c) * p.hv + h) * (kScStride * kC);
        for (int idx = tid; idx < kScStride * kC; idx += NT) sSc[idx] = SCg[idx];
        __syncthreads();

        // X = K H and Z = Q H  (contraction over dk)
        bf16x8 hb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) hb[ks] = pack8(H[2 * ks], H[2 * ks + 1]);
        f32x4 X[4], Z[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            X[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
            Z[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                X[tau] = mfma16(lds_pair(sK, SK, 16 * tau + l16, 32 * ks, g4), hb[ks], X[tau]);
                Z[tau] = mfma16(lds_pair(sQ, SK, 16 * tau + l16, 32 * ks, g4), hb[ks], Z[tau]);
            }
        }
        // Y = diag(beta) (V - diag(exp(gamma) rk) X)
        f32x4 Y[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * g4 + i;
                const float vv = bf16_to_f32(sV[r * SV + wave * 16 + l16]);
                Y[tau][i] = sSc[kC + r] * (vv - sSc[r] * X[tau][i]);
            }
        const bf16x8 yb0 = pack8(Y[0], Y[1]), yb1 = pack8(Y[2], Y[3]);
        // U = T Y   (T lower triangular: skip the all-zero upper k-step)
        f32x4 U[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            U[tau] = mfma16(lds_pair(sT, ST, 16 * tau + l16, 0, g4), yb0, f32x4{0.f, 0.f, 0.f, 0.f});
            if (tau >= 2) U[tau] = mfma16(lds_pair(sT, ST, 16 * tau + l16, 32, g4), yb1, U[tau]);
        }
        const bf16x8 ub0 = pack8(U[0], U[1]), ub1 = pack8(U[2], U[3]);
        // O = diag(exp(gamma) rq) Z + P U
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            f32x4 O = mfma16(lds_pair(sP, ST, 16 * tau + l16, 0, g4), ub0, f32x4{0.f, 0.f, 0.f, 0.f});
            if (tau >= 2) O = mfma16(lds_pair(sP, ST, 16 * tau + l16, 32, g4), ub1, O);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tau + 4 * g4 + i;
                if (r < len) {
                    const float ov = sSc[2 * kC + r] * Z[tau][i] + O[i];
                    p.o[(static_cast<size_t>(t0 + r) * p.hv + h) * p.dv + col] = f32_to_bf16(ov);
                }
            }
        }
        // H' = exp(gamma_last) H + K^T diag(rk exp(gamma_last - gamma)) U
        f32x4 DU[4];
#pragma unroll
        for (int tau = 0; tau < 4; ++tau)
#pragma unroll
            for (int i = 0; i < 4; ++i) DU[tau][i] = sSc[3 * kC + 16 * tau + 4 * g4 + i] * U[tau][i];
        const bf16x8 db0 = pack8(DU[0], DU[1]), db1 = pack8(DU[2], DU[3]);
        const float e = sSc[4 * kC];
#pragma unroll
        for (int mu = 0; mu < MT; ++mu) {
            H[mu] *= e;
            H[mu] = mfma16(lds_pair(sKt, ST, 16 * mu + l16, 0, g4), db0, H[mu]);
            H[mu] = mfma16(lds_pair(sKt, ST, 16 * mu + l16, 32, g4), db1, H[mu]);
        }
    }

    float* out = p.pool + (static_cast<size_t>(dsl) * p.hv + h) * (static_cast<size_t>(DK) * p.dv);
#pragma unroll
    for (int mu = 0; mu < MT; ++mu)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(16 * mu + 4 * g4 + i) * p.dv + col] = H[mu][i];
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return gdn::fail(GDN_E_HIP, std::string("gdn_prefill_chunked: ") + what + " launch failed: " + hipGetErrorString(e));
    return GDN_OK;
}

template <int DK>
int launch_dk(const PrefillParams& p, int n_seqs, int nw, hipStream_t s) {
    if (p.num_chunks > 0) {
        hipLaunchKernelGGL((prefill_intra_kernel<DK>), dim3(p.num_chunks, p.hv), dim3(64), 0, s, p);
        const int st = check_launch("intra-chunk");
        if (st != GDN_OK) return st;
    }
    const dim3 grid(static_cast<unsigned>(p.hv * (p.dv / (16 * nw))), static_cast<unsigned>(n_seqs));
    switch (nw) {
        case 1: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 1>), grid, dim3(64), 0, s, p); break;
        case 2: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 2>), grid, dim3(128), 0, s, p); break;
        default: hipLaunchKernelGGL((prefill_recurrent_kernel<DK, 4>), grid, dim3(256), 0, s, p); break;
    }
    return check_launch("recurrence");
}

}  // namespace

namespace gdn {

int launch_prefill(const gdn_pool* pool, const gdn_prefill_args* a, const PrefillPlan& plan, void* workspace,
                   void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    PrefillParams p;
    p.cu = a->cu_seqlens;
    p.chunk_off = reinterpret_cast<const int32_t*>(ws + plan.off_chunk_offsets);
    p.chunk_off_w = reinterpret_cast<int32_t*>(ws + plan.off_chunk_offsets);
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k);
    p.v = static_cast<const uint16_t*>(a->v);
    p.g = a->g;
    p.beta = a->beta;
    p.o = static_cast<uint16_t*>(a->o);
    p.pool = pool->storage;
    p.src = a->src_slots;
    p.dst = a->dst_slots;
    p.err = a->err_flag;
    p.kt = reinterpret_cast<uint16_t*>(ws + plan.off_kt);
    p.tp = reinterpret_cast<uint16_t*>(ws + plan.off_tp);
    p.sc = reinterpret_cast<float*>(ws + plan.off_sc);
    p.n_seqs = a->num_seqs;
    p.num_chunks = plan.num_chunks;
    p.total_tokens = a->total_tokens;
    p.hk = a->num_k_heads;
    p.hv = a->num_v_heads;
    p.group = a->num_v_heads / a->num_k_heads;
    p.dv = a->dv;
    p.num_slots = pool->num_slots;
    p.scale = a->scale;
    p.eps = a->l2_eps;

    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(64), 0, s, p);
    int st = check_launch("chunk-offset");
    if (st != GDN_OK) return st;
    const int nw = a->dv >= 64 ? 4 : a->dv / 16;
    switch (a->dk) {
        case 32: return launch_dk<32>(p, a->num_seqs, nw, s);
        case 64: return launch_dk<64>(p, a->num_seqs, nw, s);
        case 128: return launch_dk<128>(p, a->num_seqs, nw, s);
        default: return fail(GDN_E_UNSUPPORTED, "gdn_prefill_chunked: unsupported dk");
    }
}

}  // namespace gdn
